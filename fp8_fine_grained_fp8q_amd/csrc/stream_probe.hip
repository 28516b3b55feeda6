// Streaming-bandwidth probes for gfx950: what plain HBM traffic of the quantizers' shape
// reaches on the device, the ceiling their GB/s figures are read against.  Measurement
// infrastructure only (the benchmark loads it); no part of the quantization or GEMM path.
//
//   probe_copy(src, dst, n16, stream)          : dst[i] = src[i] for n16 16-byte words
//   probe_read2_write1(src, dst, n16, stream)  : reads n16 16-byte words (eight BF16 values),
//                                                writes the high byte of each value (8 bytes
//                                                per word): the quantizers' 2:1 read/write mix
//                                                with no arithmetic
//
// Each thread moves kU words: all kU loads are issued before any store, the loads carry the
// non-temporal hint the quantizers use.  Pointers are device pointers, 16-byte aligned;
// n16 > 0.  Returns the launch's hipError_t as an int.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kU = 4;
constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                        int64_t n16) {
  const int64_t base = (static_cast<int64_t>(blockIdx.x) * kU) * kThreads + threadIdx.x;
  u32x4 v[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    if (i < n16) dst[i] = v[u];
  }
}

__global__ __launch_bounds__(kThreads) void read2_write1_kernel(const u32x4 *__restrict__ src,
                                                                uint2 *__restrict__ dst, int64_t n16) {
  const int64_t base = (static_cast<int64_t>(blockIdx.x) * kU) * kThreads + threadIdx.x;
  u32x4 v[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    // high byte of each of the eight 16-bit values
    const uint32_t lo = __builtin_amdgcn_perm(v[u].y, v[u].x, 0x07050301u);
    const uint32_t hi = __builtin_amdgcn_perm(v[u].w, v[u].z, 0x07050301u);
    if (i < n16) dst[i] = make_uint2(lo, hi);
  }
}

int grid_for(int64_t n16) { return static_cast<int>((n16 + kU * kThreads - 1) / (kU * kThreads)); }

}  // namespace

extern "C" int probe_copy(const void *src, void *dst, int64_t n16, void *stream) {
  if (n16 <= 0 || n16 > (static_cast<int64_t>(1) << 34)) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n16);
  return static_cast<int>(hipGetLastError());
}

extern "C" int probe_read2_write1(const void *src, void *dst, int64_t n16, void *stream) {
  if (n16 <= 0 || n16 > (static_cast<int64_t>(1) << 34)) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(read2_write1_kernel, dim3(grid_for(n16)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), static_cast<uint2 *>(dst),
                     n16);
  return static_cast<int>(hipGetLastError());
}

// Unit-rate probes for gfx950: what one CU's LDS, its direct-to-LDS copy path and its
// matrix core deliver on their own, the rates the GEMM kernels' phases are read against.
// Measurement infrastructure only (loaded by the unit_rates module); no part of the
// quantization or GEMM path.
//
// Every probe runs one workgroup of 512 threads (8 waves) per CU: a dynamic LDS request
// (on top of the static arrays) keeps a second workgroup off the CU.  Each workgroup writes
// the shader-clock cycles (s_memtime) and the 100 MHz reference-clock ticks
// (s_memrealtime) of its timed loop to cyc[2*b] and cyc[2*b + 1], and a checksum of what it
// read to out[b*512 + tid] (so that nothing is optimised away).  All accesses stay inside
// the arrays named below; iters bounds every loop.
//
//   probe_lds_read(blocks, iters, out, cyc, stream)
//       each wave reads 8 KB per iteration with ds_read_b128, one contiguous KB per
//       instruction (lane l at byte 16*l), from a 64 KB LDS array
//   probe_lds_copy(mode, blocks, iters, src, out, cyc, stream)
//       each wave issues 8 loads of 64 lanes per iteration from a 512 KB device buffer src
//       (L2-resident after the first pass), at most 16 in flight: mode 0 buffer_load ... lds
//       with 16 bytes per lane into a 64 KB LDS array, mode 1 the same with 4 bytes per
//       lane, mode 2 16-byte loads into registers (folded into the checksum)
//   probe_lds_mix(burst, blocks, iters_r, iters_c, src, out, cyc, stream)
//       waves 0-3 read LDS in bursts of `burst` (8 or 16) one-KB ds_read_b128, each burst
//       waited for before use, while waves 4-7 copy as probe_lds_copy mode 0, into
//       separate 64 KB arrays (128 KB of static LDS: one workgroup per CU); cyc holds four
//       values per workgroup, the readers' cycles and ticks, then the copiers'
//   probe_mfma(mode, blocks, iters, out, cyc, stream)
//       v_mfma_f32_16x16x128_f8f6f4 on register operands (random finite E4M3 codes, 4 row
//       and 4 column fragments per wave): mode 0 8 MFMAs per iteration chained through C;
//       mode 1 the same plus 4 FP32 FMAs per MFMA on accumulators of their own; mode 2 16
//       MFMAs per iteration with C = 0, each result folded into an FP32 accumulator with 4
//       FMAs one fragment column (4 MFMAs) later, the GEMM's promotion pattern; mode 3 the
//       same fold issued right after its own MFMA (waiting for its result); mode 4 mode 2
//       in the GEMM's issue order (each MFMA after a group of 4 FMAs, pinned by
//       scheduling barriers)
//
// Returns the launch's hipError_t as an int (hipErrorInvalidValue for a bad argument).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kProbeThreads = 512;
// Dynamic LDS per workgroup: with the LDS probes' 64 KB static arrays 32 KB, for the MFMA
// probe (no static LDS) 96 KB, so that two workgroups never fit the CU's 160 KB.
constexpr size_t kPadLdsProbe = 32 * 1024;
constexpr size_t kPadMfmaProbe = 96 * 1024;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define PROBE_LDS __attribute__((address_space(3)))

__device__ __forceinline__ void record(unsigned long long *cyc, unsigned long long t0, unsigned long long r0) {
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    cyc[2 * blockIdx.x] = t1 - t0;
    cyc[2 * blockIdx.x + 1] = r1 - r0;
  }
}

__global__ __launch_bounds__(kProbeThreads) void lds_read_kernel(uint32_t *out, unsigned long long *cyc, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];  // 64 KB
  extern __shared__ uint32_t pad[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 16384; i += kProbeThreads) buf[i] = i * 2654435761u;
  if (tid == 0) pad[0] = 1;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc0 = 0x03020100u, acc1 = 0x07060504u;
  // bytes 16*(64*wave + lane) + 1024*u, u < 8: below 24 KB
  const char *base = reinterpret_cast<const char *>(buf) + (wave * 64 + lane) * 16;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const uint4 a = *reinterpret_cast<const uint4 *>(base + u * 1024);
      const uint4 b = *reinterpret_cast<const uint4 *>(base + (u + 1) * 1024);
      acc0 = __builtin_amdgcn_perm(a.x ^ a.y, a.z ^ a.w, acc0);
      acc1 = __builtin_amdgcn_perm(b.x ^ b.y, b.z ^ b.w, acc1);
    }
  }
  __syncthreads();
  record(cyc, t0, r0);
  out[blockIdx.x * kProbeThreads + tid] = acc0 ^ acc1;
}

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void lds_copy_kernel(const uint8_t *src, uint32_t *out,
                                                                 unsigned long long *cyc, int iters) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[65536];
  extern __shared__ uint32_t pad[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) pad[0] = 1;
  for (int i = tid; i < 16384; i += kProbeThreads) reinterpret_cast<uint32_t *>(lds)[i] = 0u;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src), (short)0, 512 * 1024, 0x00020000);
  uint32_t acc = 0;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // source KB (8*(8*it + i) + wave) mod 512; LDS slot 8*wave + i of 64
      const int blk = ((it * 8 + i) * 8 + wave) & 511;
      if (MODE == 0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PROBE_LDS void *)(lds + (8 * wave + i) * 1024), 16, lane * 16,
                                                 blk * 1024, 0, 0);
      } else if (MODE == 1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PROBE_LDS void *)(lds + (8 * wave + i) * 1024), 4, lane * 4,
                                                 blk * 1024, 0, 0);
      } else {
        const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, blk * 1024, 0);
        acc ^= static_cast<uint32_t>(v[0] ^ v[1] ^ v[2] ^ v[3]);
      }
    }
    if (MODE <= 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  record(cyc, t0, r0);
  out[blockIdx.x * kProbeThreads + tid] = acc ^ reinterpret_cast<const uint32_t *>(lds)[tid];
}

// Waves 0-3 read LDS as lds_read_kernel does (from one 64 KB array) while waves 4-7 copy
// into another 64 KB array as lds_copy_kernel<0> does; each half times its own loop
// (readers: cyc[4b], cyc[4b+1]; copiers: cyc[4b+2], cyc[4b+3]).  iters_r or iters_c = 0
// leaves that half idle.
template <int BURST>
__global__ __launch_bounds__(kProbeThreads) void lds_mix_kernel(const uint8_t *src, uint32_t *out,
                                                                unsigned long long *cyc, int iters_r, int iters_c) {
  __shared__ __attribute__((aligned(16))) uint32_t rbuf[16384];  // 64 KB read by waves 0-3
  __shared__ __attribute__((aligned(1024))) uint8_t cbuf[65536];  // 64 KB written by waves 4-7
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 16384; i += kProbeThreads) {
    rbuf[i] = i * 2654435761u;
    reinterpret_cast<uint32_t *>(cbuf)[i] = 0u;
  }
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src), (short)0, 512 * 1024, 0x00020000);
  uint32_t acc0 = 0x03020100u, acc1 = 0x07060504u;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  if (wave < 4) {
    // BURST reads of one KB each, all issued before the first is used (a memory phase's
    // pattern); bytes 16*(64*wave + lane) + 1024*u, u < BURST: below 20 KB
    const char *base = reinterpret_cast<const char *>(rbuf) + (wave * 64 + lane) * 16;
    for (int it = 0; it < iters_r; ++it) {
      asm volatile("" ::: "memory");
      uint4 v[BURST];
#pragma unroll
      for (int u = 0; u < BURST; ++u) v[u] = *reinterpret_cast<const uint4 *>(base + u * 1024);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < BURST; u += 2) {
        acc0 = __builtin_amdgcn_perm(v[u].x ^ v[u].y, v[u].z ^ v[u].w, acc0);
        acc1 = __builtin_amdgcn_perm(v[u + 1].x ^ v[u + 1].y, v[u + 1].z ^ v[u + 1].w, acc1);
      }
    }
  } else {
    const int cw = wave - 4;  // copier 0..3: LDS slots 16*cw + i of 64
    for (int it = 0; it < iters_c; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int blk = ((it * 8 + i) * 4 + cw) & 511;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PROBE_LDS void *)(cbuf + (16 * cw + 2 * i + (it & 1)) * 1024), 16,
                                                 lane * 16, blk * 1024, 0, 0);
      }
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0 && (wave == 0 || wave == 4)) {
    const int o = wave == 0 ? 0 : 2;
    cyc[4 * blockIdx.x + o] = t1 - t0;
    cyc[4 * blockIdx.x + o + 1] = r1 - r0;
  }
  __syncthreads();
  out[blockIdx.x * kProbeThreads + tid] = acc0 ^ acc1 ^ reinterpret_cast<const uint32_t *>(cbuf)[tid];
}

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void mfma_kernel(uint32_t *out, unsigned long long *cyc, int iters) {
  extern __shared__ uint32_t pad[];
  const int tid = threadIdx.x;
  if (tid == 0) pad[0] = 1;
  // finite E4M3 codes (exponent field 1..14) from a lane hash: 4 row and 4 column fragments
  i32x8 xa[4], wb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = ((tid * 8 + i) * 4 + f) * 2654435761u + 12345u;
      xa[f][i] = static_cast<int>((h & 0x87878787u) | 0x08080808u);
      const uint32_t g = ((tid * 8 + i) * 4 + f) * 2246822519u + 7u;
      wb[f][i] = static_cast<int>((g & 0x87878787u) | 0x10101010u);
    }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4][4], pp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    pp[f] = zero;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[f][j] = zero;
  }
  float d[32], s[4];
#pragma unroll
  for (int e = 0; e < 32; ++e) d[e] = tid * 1e-3f + e;
#pragma unroll
  for (int f = 0; f < 4; ++f) s[f] = (1.0f + 0.125f * f + tid * 1e-6f) / (1 << 20);
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (MODE == 0 || MODE == 1) {
      // 8 MFMAs per iteration, chained through C in 8 accumulators (acc[f][j], j < 2)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f32x4 &cq = acc[q & 3][q >> 2];
        cq = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[q >> 2], xa[q & 3], cq, 0, 0, 0, 0, 0, 0);
        if (MODE == 1) {
          // 4 FMAs on accumulators of their own, each updated once per iteration
#pragma unroll
          for (int e = 0; e < 4; ++e) d[4 * q + e] = __builtin_fmaf(d[4 * q + e], s[e], s[(e + 1) & 3]);
        }
      }
    } else {
      // 16 MFMAs per iteration: 4 fragment columns j x 4 fragment rows f, C = 0
      xa[0][0] ^= it & 0x01010101;  // a new product every iteration (one integer op per 16 MFMAs)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (MODE == 2 || MODE == 4) {
            // the GEMM's pattern: fold column j - 1's partial of row f, then its MFMA for column j
            const int jp = (j + 3) & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[f][jp][e] = __builtin_fmaf(pp[f][e], s[f], acc[f][jp][e]);
            pp[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[j], xa[f], zero, 0, 0, 0, 0, 0, 0);
          } else {
            const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[j], xa[f], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[f][j][e] = __builtin_fmaf(p[e], s[f], acc[f][j][e]);
          }
        }
        if (MODE == 4) {
          // the GEMM's issue order: each MFMA after a group of 4 promotion FMAs
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  __syncthreads();
  record(cyc, t0, r0);
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) sum += d[e];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    sum += pp[f][0] + pp[f][1] + pp[f][2] + pp[f][3];
#pragma unroll
    for (int j = 0; j < 4; ++j) sum += acc[f][j][0] + acc[f][j][1] + acc[f][j][2] + acc[f][j][3];
  }
  out[blockIdx.x * kProbeThreads + tid] = __float_as_uint(sum);
}

template <class Kern, class... Args>
int launch_probe(Kern kern, size_t pad, int blocks, hipStream_t stream, Args... args) {
  if (blocks <= 0 || blocks > 65536) return static_cast<int>(hipErrorInvalidValue);
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(pad));
  if (e != hipSuccess) return static_cast<int>(e);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kProbeThreads), pad, stream, args...);
  return static_cast<int>(hipGetLastError());
}

bool iters_ok(int iters) { return iters > 0 && iters <= (1 << 24); }

}  // namespace

extern "C" int probe_lds_read(int blocks, int iters, void *out, void *cyc, void *stream) {
  if (!iters_ok(iters)) return static_cast<int>(hipErrorInvalidValue);
  return launch_probe(lds_read_kernel, kPadLdsProbe, blocks, static_cast<hipStream_t>(stream),
                      static_cast<uint32_t *>(out), static_cast<unsigned long long *>(cyc), iters);
}

extern "C" int probe_lds_copy(int mode, int blocks, int iters, const void *src, void *out, void *cyc,
                              void *stream) {
  if (!iters_ok(iters)) return static_cast<int>(hipErrorInvalidValue);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t *p = static_cast<const uint8_t *>(src);
  uint32_t *o = static_cast<uint32_t *>(out);
  unsigned long long *c = static_cast<unsigned long long *>(cyc);
  switch (mode) {
    case 0: return launch_probe(lds_copy_kernel<0>, kPadLdsProbe, blocks, s, p, o, c, iters);
    case 1: return launch_probe(lds_copy_kernel<1>, kPadLdsProbe, blocks, s, p, o, c, iters);
    case 2: return launch_probe(lds_copy_kernel<2>, kPadLdsProbe, blocks, s, p, o, c, iters);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

extern "C" int probe_lds_mix(int burst, int blocks, int iters_r, int iters_c, const void *src, void *out,
                             void *cyc, void *stream) {
  if (iters_r < 0 || iters_c < 0 || iters_r > (1 << 24) || iters_c > (1 << 24) || iters_r + iters_c == 0)
    return static_cast<int>(hipErrorInvalidValue);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t *p = static_cast<const uint8_t *>(src);
  uint32_t *o = static_cast<uint32_t *>(out);
  unsigned long long *c = static_cast<unsigned long long *>(cyc);
  if (burst == 8) return launch_probe(lds_mix_kernel<8>, size_t(0), blocks, s, p, o, c, iters_r, iters_c);
  if (burst == 16) return launch_probe(lds_mix_kernel<16>, size_t(0), blocks, s, p, o, c, iters_r, iters_c);
  return static_cast<int>(hipErrorInvalidValue);
}

extern "C" int probe_mfma(int mode, int blocks, int iters, void *out, void *cyc, void *stream) {
  if (!iters_ok(iters)) return static_cast<int>(hipErrorInvalidValue);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t *o = static_cast<uint32_t *>(out);
  unsigned long long *c = static_cast<unsigned long long *>(cyc);
  switch (mode) {
    case 0: return launch_probe(mfma_kernel<0>, kPadMfmaProbe, blocks, s, o, c, iters);
    case 1: return launch_probe(mfma_kernel<1>, kPadMfmaProbe, blocks, s, o, c, iters);
    case 2: return launch_probe(mfma_kernel<2>, kPadMfmaProbe, blocks, s, o, c, iters);
    case 3: return launch_probe(mfma_kernel<3>, kPadMfmaProbe, blocks, s, o, c, iters);
    case 4: return launch_probe(mfma_kernel<4>, kPadMfmaProbe, blocks, s, o, c, iters);
  }
  return static_cast<int>(hipErrorInvalidValue);
}

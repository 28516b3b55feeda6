// Expert-parallel dispatch and combine around the grouped GEMM, one GPU's share, for gfx950.
//
// Each token is routed to 8 of 256 experts (dlbhg.com page on DeepSeek-V3's training
// techniques, section 1.1, item 2), the experts are spread over the GPUs (same page, section
// 2.1: 64-way expert parallelism) and tokens reach their experts and come back by all-to-all
// dispatch and combine (same page, section 3.1; dtcms.com page, the DualPipe paragraph).
// The exchange itself needs several GPUs; these kernels are the work on either side of it
// on the GPU that owns experts [e_begin, e_begin + E):
//   * route: from the top-k expert ids of T tokens, the expert-sorted row of every (token,
//     slot) routed to a local expert (experts in order, tokens ascending within one), the
//     per-expert offsets the grouped GEMM reads, and the inverse map for the combine;
//   * pack: copy each such row's E4M3 codes and 1x128 tile scales into that layout (the
//     activation quantizer is row-local, so quantizing before the exchange is the same as
//     after it, and the payload is the FP8 codes plus 4 bytes per 128 of them);
//   * combine: y[t] = sum over the token's local slots s of w[t, s] * out[row(t, s)], FP32
//     accumulation in slot order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_launch.h"

namespace fp8q {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxLocalExperts = 1024;
constexpr int kBatch = 16;  // 64-entry chunks whose id loads a wave issues together

// Count of the set bits of mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

// One workgroup.  Wave w owns the (token, slot) entries [w*per, (w+1)*per) of ids[T*k] in
// order.  1: per-wave, per-expert counts (LDS atomics).  2: one thread per expert sums the
// waves' counts; a serial scan gives the offsets and each wave's first row per expert.
// 3: each wave walks its entries again, 64 at a time: the lanes of one expert (found with a
// ballot) take consecutive rows after that expert's running count, lower lanes first, so
// rows follow the entry order, i.e. token order within an expert.  A wave reads the ids of
// kBatch chunks at once; its running counts live in a register for up to 64 experts.
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                                  int k, int64_t e_begin, int E, int64_t cap,
                                                                  int32_t *__restrict__ offsets,
                                                                  int32_t *__restrict__ token_row,
                                                                  int32_t *__restrict__ row_token) {
  __shared__ int32_t cnt[kRouteWaves * kMaxLocalExperts];  // counts, then running rows
  __shared__ int32_t tot[kMaxLocalExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per = ((n + kRouteWaves - 1) / kRouteWaves + 63) / 64 * 64;
  const int64_t lo = wave * per, hi = lo + per < n ? lo + per : n;
  auto local_expert = [&](int64_t idx) -> int {
    if (idx >= hi) return -1;
    const int64_t g = static_cast<int64_t>(ids[idx]) - e_begin;
    return g >= 0 && g < E ? static_cast<int>(g) : -1;
  };
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) cnt[i] = 0;
  __syncthreads();
  // The id loads of kBatch chunks are issued together (one wave walks its range serially).
  for (int64_t c0 = lo; c0 < hi; c0 += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) eb[b] = local_expert(c0 + 64 * b + lane);
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (eb[b] >= 0) atomicAdd(&cnt[wave * E + eb[b]], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    int s = 0;
    for (int w = 0; w < kRouteWaves; ++w) s += cnt[w * E + e];
    tot[e] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      const int t = tot[e];
      tot[e] = run;
      run += t;
    }
    offsets[E] = run;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {  // each wave's first row of expert e
    int base = tot[e];
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = base;
      base += c;
    }
  }
  __syncthreads();
  // Up to 64 local experts: lane e of each wave keeps the wave's running row of expert e in
  // a register, so ranking a chunk needs no LDS traffic (readlane of uniform lanes only).
  const bool in_regs = E <= 64;
  int run = in_regs && lane < E ? cnt[wave * E + lane] : 0;
  for (int64_t c0 = lo; c0 < hi; c0 += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) eb[b] = local_expert(c0 + 64 * b + lane);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {  // chunks in entry order
      const int64_t idx = c0 + 64 * b + lane;
      const int e = eb[b];
      int row = -1;
      uint64_t pending = __ballot(e >= 0);
      while (pending != 0) {
        const int leader = __ffsll(static_cast<long long>(pending)) - 1;
        const int ee = __builtin_amdgcn_readlane(e, leader);
        const uint64_t m = __ballot(e == ee);
        if (in_regs) {
          const int r0 = __builtin_amdgcn_readlane(run, ee);
          if (e == ee) row = r0 + lanes_below(m);
          if (lane == ee) run = r0 + __popcll(m);
        } else {
          const int r0 = cnt[wave * E + ee];
          if (e == ee) row = r0 + lanes_below(m);
          if (lane == leader) cnt[wave * E + ee] = r0 + __popcll(m);
        }
        pending &= ~m;
      }
      // rows past the capacity are dropped (their slots read as not local); offsets still
      // count them, so the caller can see that the capacity was too small
      if (idx < hi) token_row[idx] = row < cap ? row : -1;
      if (row >= 0 && row < cap) row_token[row] = static_cast<int32_t>(idx / k);
    }
  }
}

// One wave per dispatched row r < offsets[E]: the token's K code bytes (16 per lane and
// step) and its K/128 tile scales (sa[kb][t] -> sa_s[kb][r], row stride `cap`).
__global__ __launch_bounds__(256) void moe_pack_kernel(const uint8_t *__restrict__ xq, const float *__restrict__ sa,
                                                       int64_t T, int64_t K, const int32_t *__restrict__ row_token,
                                                       const int32_t *__restrict__ offsets, int E, int64_t cap,
                                                       uint8_t *__restrict__ xq_s, float *__restrict__ sa_s) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= offsets[E] || r >= cap) return;
  const int64_t t = row_token[r];
  const uint4 *src = reinterpret_cast<const uint4 *>(xq + t * K);
  uint4 *dst = reinterpret_cast<uint4 *>(xq_s + r * K);
  for (int64_t i = lane; i < K / 16; i += 64) dst[i] = src[i];
  for (int64_t kb = lane; kb < K / 128; kb += 64) sa_s[kb * cap + r] = sa[kb * T + t];
}

template <bool kInF32>
__device__ __forceinline__ void load8(const void *p, int64_t off, float (&v)[8]) {
  if (kInF32) {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + off);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// One workgroup per token; each thread takes 8 consecutive columns at a time.  The slots
// are visited in order and each adds w * out[row] with one FMA per element.
template <bool kInF32, bool kOutF32>
__global__ __launch_bounds__(256) void moe_combine_kernel(const void *__restrict__ out, int64_t N,
                                                          const int32_t *__restrict__ token_row,
                                                          const float *__restrict__ w, int k, int64_t cap,
                                                          void *__restrict__ y) {
  const int64_t t = blockIdx.x;
  for (int64_t c = threadIdx.x; c < N / 8; c += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < k; ++s) {
      const int32_t r = token_row[t * k + s];
      if (r < 0 || r >= cap) continue;  // not a local slot (or not a row of `out`)
      const float ws = w[t * k + s];
      float v[8];
      load8<kInF32>(out, static_cast<int64_t>(r) * N + 8 * c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(ws, v[i], acc[i]);
    }
    if (kOutF32) {
      float *yo = static_cast<float *>(y) + t * N + 8 * c;
      *reinterpret_cast<float4 *>(yo) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4 *>(yo + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u = __float_as_uint(acc[i]);
        b[i] = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
      }
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + t * N + 8 * c) =
          make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
    }
  }
}

hipError_t launch_moe_dispatch(const int32_t *ids, int64_t T, int64_t k, int64_t e_begin, int64_t E,
                               const uint8_t *xq, const float *sa, int64_t K, int64_t cap, uint8_t *xq_s,
                               float *sa_s, int32_t *offsets, int32_t *token_row, int32_t *row_token,
                               hipStream_t stream) {
  if (E < 1 || E > kMaxLocalExperts || (cap + 3) / 4 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, ids, T * k, static_cast<int>(k),
                     e_begin, static_cast<int>(E), cap, offsets, token_row, row_token);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || cap == 0) return e;
  hipLaunchKernelGGL(moe_pack_kernel, dim3(static_cast<uint32_t>((cap + 3) / 4)), dim3(256), 0, stream, xq, sa, T,
                     K, row_token, offsets, static_cast<int>(E), cap, xq_s, sa_s);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void *out, bool in_f32, int64_t cap, int64_t N, const int32_t *token_row,
                              const float *w, int64_t T, int64_t k, void *y, bool out_f32, hipStream_t stream) {
  if (T > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(T)), block(256);
  const int kk = static_cast<int>(k);
  if (in_f32 && out_f32)
    hipLaunchKernelGGL((moe_combine_kernel<true, true>), grid, block, 0, stream, out, N, token_row, w, kk, cap, y);
  else if (in_f32)
    hipLaunchKernelGGL((moe_combine_kernel<true, false>), grid, block, 0, stream, out, N, token_row, w, kk, cap, y);
  else if (out_f32)
    hipLaunchKernelGGL((moe_combine_kernel<false, true>), grid, block, 0, stream, out, N, token_row, w, kk, cap, y);
  else
    hipLaunchKernelGGL((moe_combine_kernel<false, false>), grid, block, 0, stream, out, N, token_row, w, kk, cap, y);
  return hipGetLastError();
}

}  // namespace fp8q

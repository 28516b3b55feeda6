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
constexpr int64_t kChunk = 1024;  // (token, slot) entries per routing workgroup; >= kMaxLocalExperts

// Count of the set bits of mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

// The routing splits the n = T*k entries into C = max(1, floor(n / kChunk)) chunks of
// kChunk entries in order, the last one taking the remainder (so every chunk but a lone one
// holds at least kChunk >= E entries).  Entry range of chunk c:
__device__ __forceinline__ void chunk_range(int64_t c, int64_t C, int64_t n, int64_t &lo, int64_t &hi) {
  lo = c * kChunk;
  hi = c == C - 1 ? n : lo + kChunk;
}

__device__ __forceinline__ int local_expert(const int32_t *__restrict__ ids, int64_t idx, int64_t hi,
                                            int64_t e_begin, int E) {
  if (idx >= hi) return -1;
  const int64_t g = static_cast<int64_t>(ids[idx]) - e_begin;
  return g >= 0 && g < E ? static_cast<int>(g) : -1;
}

// Exclusive prefix sum of v over the kRouteThreads threads in thread order; *total gets the
// sum.  Every thread of the workgroup calls it; ws is kRouteWaves ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int *ws, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d);
    if (lane >= d) inc += u;
  }
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kRouteWaves; ++w) {
    const int t = ws[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();  // ws may be reused after this
  *total = all;
  return before + inc - v;
}

// 1 (C > 1 only): each workgroup counts its chunk's entries per local expert and leaves the
// counts in the first E entries of its own range of token_row, which the ranking pass
// overwrites later (only this chunk's workgroups ever touch that range).
__global__ __launch_bounds__(kRouteThreads) void moe_count_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                                  int64_t C, int64_t e_begin, int E,
                                                                  int32_t *__restrict__ token_row) {
  __shared__ int32_t hist[kMaxLocalExperts];
  int64_t lo, hi;
  chunk_range(blockIdx.x, C, n, lo, hi);
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  for (int64_t i = lo + threadIdx.x; i < hi; i += kRouteThreads) {
    const int e = local_expert(ids, i, hi, e_begin, E);
    if (e >= 0) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) token_row[lo + e] = hist[e];
}

// 2 (C > 1 only), one workgroup: offsets[e] = rows of the experts before e, and in place of
// chunk c's count of expert e, that chunk's first row of expert e (offsets[e] plus the counts
// of the earlier chunks).  Thread (g, e) = (tid / E, tid % E) walks a contiguous run of
// chunks for expert e; the runs' sums are scanned per expert, the experts' totals over the
// workgroup.
__global__ __launch_bounds__(kRouteThreads) void moe_scan_kernel(int64_t n, int64_t C, int E,
                                                                 int32_t *__restrict__ offsets,
                                                                 int32_t *__restrict__ token_row) {
  __shared__ int32_t part[kRouteThreads];
  __shared__ int32_t first[kMaxLocalExperts];
  __shared__ int32_t ws[kRouteWaves];
  const int tid = threadIdx.x;
  const int G = kRouteThreads / E;
  const int64_t per = (C + G - 1) / G;
  const int g = tid / E, e = tid % E;
  const int64_t c_lo = g < G ? g * per : C, c_hi = c_lo + per < C ? c_lo + per : C;
  int s = 0;
#pragma unroll 8
  for (int64_t c = c_lo; c < c_hi; ++c) s += token_row[c * kChunk + e];  // independent loads
  if (g < G) part[tid] = s;
  __syncthreads();
  int tot = 0;
  if (tid < E) {
    for (int j = 0; j < G; ++j) {  // runs before g, per expert
      const int p = part[j * E + tid];
      part[j * E + tid] = tot;
      tot += p;
    }
  }
  int all;
  const int ex = block_exclusive_scan(tid < E ? tot : 0, ws, &all);
  if (tid < E) {
    offsets[tid] = ex;
    first[tid] = ex;
  }
  if (tid == 0) offsets[E] = all;
  __syncthreads();
  int base = g < G ? first[e] + part[tid] : 0;
#pragma unroll 8
  for (int64_t c = c_lo; c < c_hi; ++c) {
    const int v = token_row[c * kChunk + e];
    token_row[c * kChunk + e] = base;
    base += v;
  }
}

// 3: each workgroup ranks its chunk, 1024 entries per round, one per thread.  Within a wave
// the lanes of one expert are found without a loop: the ballots of the expert index's bits
// (and of "local") intersect to the set of lanes with this lane's expert.  A lane's row is
// the chunk's running row of its expert, plus that expert's entries in the earlier waves of
// the round, plus those in lower lanes, so rows follow entry order, i.e. token order within
// an expert.  With a lone chunk (C == 1) the workgroup counts and scans by itself and writes
// the offsets.
__global__ __launch_bounds__(kRouteThreads) void moe_rank_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                                 int64_t C, int k, int64_t e_begin, int E,
                                                                 int64_t cap, int32_t *__restrict__ offsets,
                                                                 int32_t *__restrict__ token_row,
                                                                 int32_t *__restrict__ row_token) {
  __shared__ int32_t run[kMaxLocalExperts];                  // the chunk's next row, per expert
  __shared__ int32_t wcnt[kRouteWaves * kMaxLocalExperts];   // a round's count per wave and expert
  __shared__ int32_t ws[kRouteWaves];
  const int tid = threadIdx.x, wave = tid >> 6;
  int64_t lo, hi;
  chunk_range(blockIdx.x, C, n, lo, hi);
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wcnt[i] = 0;
  if (C > 1) {
    for (int e = tid; e < E; e += kRouteThreads) run[e] = token_row[lo + e];
  } else {
    for (int e = tid; e < E; e += kRouteThreads) run[e] = 0;
    __syncthreads();
    for (int64_t i = lo + tid; i < hi; i += kRouteThreads) {
      const int e = local_expert(ids, i, hi, e_begin, E);
      if (e >= 0) atomicAdd(&run[e], 1);
    }
    __syncthreads();
    int all;
    const int cnt = tid < E ? run[tid] : 0;
    const int ex = block_exclusive_scan(cnt, ws, &all);
    if (tid < E) {
      run[tid] = ex;
      offsets[tid] = ex;
    }
    if (tid == 0) offsets[E] = all;
  }
  __syncthreads();  // the counts in token_row are read before this chunk's rows overwrite them
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int64_t r0 = lo; r0 < hi; r0 += kRouteThreads) {
    const int64_t idx = r0 + tid;
    const int e = local_expert(ids, idx, hi, e_begin, E);
    uint64_t m = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bit = __ballot(e >= 0 && ((e >> b) & 1));
      m &= ((e >> b) & 1) ? bit : ~bit;
    }
    const bool leader = e >= 0 && lanes_below(m) == 0;
    if (leader) wcnt[wave * E + e] = __popcll(m);
    __syncthreads();
    int row = -1, last_wave = -1, round_total = 0;
    if (e >= 0) {
      int before = 0;
#pragma unroll
      for (int w = 0; w < kRouteWaves; ++w) {
        const int t = wcnt[w * E + e];
        before += w < wave ? t : 0;
        round_total += t;
        last_wave = t > 0 ? w : last_wave;
      }
      row = run[e] + before + lanes_below(m);
    }
    __syncthreads();  // every lane has read run[] and wcnt[]
    if (leader) {
      wcnt[wave * E + e] = 0;
      if (last_wave == wave) run[e] += round_total;
    }
    // rows past the capacity are dropped (their slots read as not local); offsets still count
    // them, so the caller can see that the capacity was too small
    if (idx < hi) token_row[idx] = row < cap ? row : -1;
    if (row >= 0 && row < cap) row_token[row] = static_cast<int32_t>(idx / k);
    __syncthreads();
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
  const int64_t n = T * k, C = n / kChunk > 1 ? n / kChunk : 1;
  if (C > 0x7fffffff) return hipErrorInvalidValue;
  const int kk = static_cast<int>(k), EE = static_cast<int>(E);
  if (C > 1) {
    hipLaunchKernelGGL(moe_count_kernel, dim3(static_cast<uint32_t>(C)), dim3(kRouteThreads), 0, stream, ids, n, C,
                       e_begin, EE, token_row);
    hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(kRouteThreads), 0, stream, n, C, EE, offsets, token_row);
  }
  hipLaunchKernelGGL(moe_rank_kernel, dim3(static_cast<uint32_t>(C)), dim3(kRouteThreads), 0, stream, ids, n, C, kk,
                     e_begin, EE, cap, offsets, token_row, row_token);
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

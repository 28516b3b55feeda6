// Online fine-grained E4M3 quantizers for gfx950.
//
// Activation tiles are 1x128 (one row, 128 consecutive K) and weight blocks 128x128, each
// with its own FP32 scale amax/448 taken from the group's current values: codingmall.com
// page on FP8 in DeepSeek-V3 training, sections "Dinh luong hat min" and "Dinh luong truc
// tuyen"; risenshineclean.com DeepSeek training-algorithm page, section 3 (1x128 tile =
// one token's 128 channels; scales computed online, no delayed scaling).
//
// Both kernels are HBM-bound: each reads 2 bytes and writes 1 byte per element.  Loads are
// 16-byte per lane, so one 1x128 BF16 tile (256 B) is exactly one 16-lane DPP row and its
// amax reduces with four row_ror steps and no LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_device.h"
#include "fp8q_launch.h"

namespace fp8q {

// ---------------------------------------------------------------------------------------
// Activation quantizer.  One wave handles a slab of 4*NR rows x 128*NK columns: lane
// (grp = lane/16, sub = lane%16) holds the 16-byte chunk `sub` of rows row0 + 4*i + grp
// (i < NR) in K blocks kb0 + k (k < NK), so each 1x128 tile is one 16-lane DPP row and
// its amax reduces with four row_ror steps and no LDS.  All NR*NK loads are issued before
// any conversion.  Consecutive waves take consecutive K-block groups of the same rows, so
// a 256-thread workgroup streams 4*NR rows x 4*NK*128 contiguous BF16 columns.  The 4*NR
// scales of a tile column are one contiguous run of sa[kb][.].
// ---------------------------------------------------------------------------------------
#ifndef FP8Q_ACT_NR
#define FP8Q_ACT_NR 2
#endif
#ifndef FP8Q_ACT_NK
#define FP8Q_ACT_NK 2
#endif
#ifndef FP8Q_ACT_NT
#define FP8Q_ACT_NT 1
#endif
constexpr int kActWavesPerBlock = 4;

// The activation quantizer's work for workgroup `block` (of act_blocks(M, K) in all).
template <int NR, int NK>
__device__ __forceinline__ void quant_act_block(int64_t block, const uint16_t *__restrict__ x, int64_t M,
                                                int64_t K, uint8_t *__restrict__ xq, float *__restrict__ sa) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = block * kActWavesPerBlock + (threadIdx.x >> 6);
  const int64_t KB = K >> 7;
  const int64_t KG = (KB + NK - 1) / NK;  // K-block groups per row slab
  const int64_t kb0 = (wave % KG) * NK;
  const int64_t row0 = (wave / KG) * (4 * NR);
  if (row0 >= M) return;
  const int grp = lane >> 4;
  const int sub = lane & 15;

  uint4 v[NK][NR];
#pragma unroll
  for (int k = 0; k < NK; ++k)
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t row = row0 + 4 * i + grp;
      const int64_t col = (kb0 + k) * 128 + sub * 8;
      if (row < M && kb0 + k < KB) {
        v[k][i] = FP8Q_ACT_NT ? load16_stream(x + row * K + col) : *reinterpret_cast<const uint4 *>(x + row * K + col);
      } else {
        v[k][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    if (kb0 + k >= KB) break;
    float scale[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float amax = row16_max(absmax8(v[k][i]));
      scale[i] = amax / kE4M3Max;  // IEEE division (correctly rounded)
    }
    const int64_t col = (kb0 + k) * 128 + sub * 8;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t row = row0 + 4 * i + grp;
      const GroupDiv dv(scale[i]);
      const uint2 q = quant8(v[k][i], dv);
      if (row < M) *reinterpret_cast<uint2 *>(xq + row * K + col) = q;
    }
    // lanes sub < NR of each DPP row store the scales of rows row0 + 4*sub + grp
    if (sub < NR) {
      float s = scale[0];
#pragma unroll
      for (int i = 1; i < NR; ++i) s = sub == i ? scale[i] : s;
      const int64_t row = row0 + 4 * sub + grp;
      if (row < M) sa[(kb0 + k) * M + row] = s;
    }
  }
}

template <int NR, int NK>
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(const uint16_t *__restrict__ x,
                                                              int64_t M, int64_t K,
                                                              uint8_t *__restrict__ xq,
                                                              float *__restrict__ sa) {
  quant_act_block<NR, NK>(blockIdx.x, x, M, K, xq, sa);
}

// Workgroups of the activation quantizer for X[M][K].
int64_t act_blocks(int64_t M, int64_t K) {
  constexpr int NR = FP8Q_ACT_NR, NK = FP8Q_ACT_NK;
  const int64_t KB = K / 128;
  const int64_t waves = ((M + 4 * NR - 1) / (4 * NR)) * ((KB + NK - 1) / NK);
  return (waves + kActWavesPerBlock - 1) / kActWavesPerBlock;
}

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sa,
                            hipStream_t stream) {
  constexpr int NR = FP8Q_ACT_NR, NK = FP8Q_ACT_NK;
  const int64_t blocks = act_blocks(M, K);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_act_1x128_kernel<NR, NK>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     stream, x, M, K, xq, sa);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Weight quantizer.  One 256-thread workgroup per 128x128 block: thread t holds chunk
// t%16 of rows t/16 + 16*i, i = 0..7 (64 values in registers).  amax: DPP inside each
// 16-lane row, readlane across the wave's four rows, LDS across the four waves.  The whole
// block shares one scale, so the division path is uniform.
//
// With kTrans the block's codes are also written transposed (W^T[K][N] codes and the
// block scale at [kb][nb]), the operand layout of the data-gradient GEMM dX = dY W: the
// codes go through a 16 KB LDS tile and each thread turns four 4x4 byte squares around
// with byte permutes, producing 16 consecutive N-bytes of four W^T rows.
// ---------------------------------------------------------------------------------------

// Byte transpose of a 4x4 square held as four dwords r0..r3 (row i = dword i, column j =
// byte j): c[j] gets byte j of r0, r1, r2, r3 in bytes 0..3.  v_perm_b32 selects bytes
// of {S0, S1} (selector 0..3 = S1 bytes 0..3, 4..7 = S0 bytes 0..3).
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, uint32_t c[4]) {
  const uint32_t a = __builtin_amdgcn_perm(r1, r0, 0x06020400u);  // r0.b0 r1.b0 r0.b2 r1.b2
  const uint32_t b = __builtin_amdgcn_perm(r1, r0, 0x07030501u);  // r0.b1 r1.b1 r0.b3 r1.b3
  const uint32_t e = __builtin_amdgcn_perm(r3, r2, 0x06020400u);  // r2.b0 r3.b0 r2.b2 r3.b2
  const uint32_t f = __builtin_amdgcn_perm(r3, r2, 0x07030501u);  // r2.b1 r3.b1 r2.b3 r3.b3
  c[0] = __builtin_amdgcn_perm(e, a, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(f, b, 0x05040100u);
  c[2] = __builtin_amdgcn_perm(e, a, 0x07060302u);
  c[3] = __builtin_amdgcn_perm(f, b, 0x07060302u);
}

// Writes the transposed 128x128 code tile held in LDS (tile[row][col], 128-byte rows) as
// rows of dst (row stride ld bytes): dst[col][row].  Thread t covers columns 4*(t%32)+j
// (j < 4) and rows 16*(t/32) .. +15.
__device__ __forceinline__ void store_transposed_tile(const uint32_t *tile, uint8_t *__restrict__ dst,
                                                      int64_t ld, int tid) {
  const int kd = tid & 31;
  const int n0 = (tid >> 5) * 16;
  uint32_t out[4][4];  // [column j][row group g]
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t *p = tile + (n0 + 4 * g) * 32 + kd;
    uint32_t c[4];
    transpose4x4(p[0], p[32], p[64], p[96], c);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j][g] = c[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4 *>(dst + (4 * kd + j) * ld + n0) = make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]);
}

// The weight quantizer's work for block `bid` (= (g*N/128 + nb)*K/128 + kb).
template <bool kTrans>
__device__ __forceinline__ void quant_w_block(int64_t bid, const uint16_t *__restrict__ w, int64_t N, int64_t K,
                                              uint8_t *__restrict__ wq, float *__restrict__ sb,
                                              uint8_t *__restrict__ wqt, float *__restrict__ sbt) {
  __shared__ float wave_max[4];
  __shared__ __attribute__((aligned(16))) uint32_t tile[kTrans ? 128 * 32 : 1];
  const int64_t KB = K >> 7, NB = N >> 7;
  const int64_t kb = bid % KB;
  const int64_t gnb = bid / KB;  // g * NB + nb
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  const int r0 = tid >> 4;
  const int64_t base = (gnb * 128) * K + kb * 128 + sub * 8;  // row gnb*128 of the [G*N][K] view

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = load16_stream(w + base + (r0 + 16 * i) * K);
  float m = absmax8(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmaxf(m, absmax8(v[i]));
  m = row16_max(m);
  m = fmaxf(fmaxf(lane_f32(m, 0), lane_f32(m, 16)), fmaxf(lane_f32(m, 32), lane_f32(m, 48)));
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = amax / kE4M3Max;
  const GroupDiv dv(s);
  // An empty asm claiming to modify the packed values: the amax pass's widened values are
  // recomputed below (one shift or mask each) rather than held in 64 registers across the
  // barrier, so more workgroups fit per CU.
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 q = quant8(v[i], dv);
    *reinterpret_cast<uint2 *>(wq + base + (r0 + 16 * i) * K) = q;
    if (kTrans) *reinterpret_cast<uint2 *>(tile + (r0 + 16 * i) * 32 + sub * 2) = q;
  }
  if (tid == 0) sb[gnb * KB + kb] = s;
  if (kTrans) {
    const int64_t g = gnb / NB, nb = gnb % NB;
    if (tid == 0) sbt[(g * KB + kb) * NB + nb] = s;
    __syncthreads();
    store_transposed_tile(tile, wqt + (g * K + kb * 128) * N + nb * 128, N, tid);
  }
}

template <bool kTrans>
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(const uint16_t *__restrict__ w,
                                                              int64_t N, int64_t K,
                                                              uint8_t *__restrict__ wq,
                                                              float *__restrict__ sb,
                                                              uint8_t *__restrict__ wqt,
                                                              float *__restrict__ sbt) {
  quant_w_block<kTrans>(blockIdx.x, w, N, K, wq, sb, wqt, sbt);
}

// Both quantizers of a linear layer in one launch: workgroups [0, w_blocks) take the
// weight blocks, the rest the activation slabs (the shorter activation work fills the tail
// of the weight work, and the layer pays one kernel boundary instead of two).  Each
// workgroup does exactly what it does in its own kernel, so the outputs are identical.
__global__ __launch_bounds__(256) void quant_act_w_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                          uint8_t *__restrict__ xq, float *__restrict__ sa,
                                                          const uint16_t *__restrict__ w, int64_t N,
                                                          uint8_t *__restrict__ wq, float *__restrict__ sb,
                                                          int64_t K, int64_t w_blocks) {
  if (static_cast<int64_t>(blockIdx.x) < w_blocks)
    quant_w_block<false>(blockIdx.x, w, N, K, wq, sb, nullptr, nullptr);
  else
    quant_act_block<FP8Q_ACT_NR, FP8Q_ACT_NK>(blockIdx.x - w_blocks, x, M, K, xq, sa);
}

hipError_t launch_quant_act_w(const uint16_t *x, int64_t M, uint8_t *xq, float *sa, const uint16_t *w, int64_t G,
                              int64_t N, uint8_t *wq, float *sb, int64_t K, hipStream_t stream) {
  const int64_t wb = G * (N / 128) * (K / 128);
  const int64_t total = wb + act_blocks(M, K);
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_w_kernel, dim3(static_cast<uint32_t>(total)), dim3(256), 0, stream, x, M, xq, sa, w,
                     N, wq, sb, K, wb);
  return hipGetLastError();
}

hipError_t launch_quant_w(const uint16_t *w, int64_t G, int64_t N, int64_t K, uint8_t *wq, float *sb,
                          uint8_t *wqt, float *sbt, hipStream_t stream) {
  const int64_t blocks = G * (N / 128) * (K / 128);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (wqt != nullptr)
    hipLaunchKernelGGL(quant_w_128x128_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       w, N, K, wq, sb, wqt, sbt);
  else
    hipLaunchKernelGGL(quant_w_128x128_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       w, N, K, wq, sb, static_cast<uint8_t *>(nullptr), static_cast<float *>(nullptr));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Activation quantizer in both orientations, for a layer whose input is needed by the
// forward GEMM (tiles of 128 along K) and by the weight-gradient GEMM dW = dY^T X, whose
// contraction runs over the tokens (tiles of 128 consecutive tokens of one channel, codes
// stored channel-major as X^T[K][M]).  One 256-thread workgroup per 128x128 block of
// X[M][K], the same register layout as the weight quantizer: thread t holds chunk t%16
// (8 columns) of rows t/16 + 16*i.  Row tiles reduce inside a DPP row as in the 1x128
// quantizer; column tiles reduce over the thread's 8 rows, across the wave with two
// lane swaps and across the waves through LDS, where 128 threads also form the column
// scales and reciprocals once.  The column codes are transposed through LDS like W^T.
// The token count M must be a multiple of 128.
// ---------------------------------------------------------------------------------------

// y = RN32(x / s) of a BF16 value x for a divisor held as (s, r, mode) in the GroupDiv
// convention.
__device__ __forceinline__ float div_any(float x, float s, float r, int mode) {
  if (mode == 1) {
    GroupDiv d(0.0f);
    d.s = s;
    d.r = r;
    return d.fast_bf16(x);
  }
  return mode == 2 ? x / s : x;
}

__device__ __forceinline__ float bf16_elem(const uint4 &v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

__global__ __launch_bounds__(256) void quant_act_dual_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                             int64_t K, uint8_t *__restrict__ xq,
                                                             float *__restrict__ sa,
                                                             uint8_t *__restrict__ xqt,
                                                             float *__restrict__ sat) {
  __shared__ float colmax[4][128];
  __shared__ float colscale[128], colrcp[128];
  __shared__ int colmode[128];
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * 32];
  const int64_t KB = K >> 7;
  const int64_t kb = blockIdx.x % KB;
  const int64_t mb = blockIdx.x / KB;
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  const int r0 = tid >> 4;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t base = (mb * 128) * K + kb * 128 + sub * 8;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = load16_stream(x + base + (r0 + 16 * i) * K);
  // values stay packed (two BF16 per register) and are widened where used: one shift or
  // mask each, which keeps the kernel small enough for 8 workgroups per CU
  auto xv = [&](int i, int e) { return bf16_elem(v[i], e); };
  // An empty asm that claims to modify the packed words: the widened values of one phase
  // then cannot be kept for the next one, and are recomputed (one shift or mask each)
  // instead of taking 64 registers across the phases.
  auto fence_values = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
  };

  // Row tiles (1x128 along K): the forward codes.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float xr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xr[e] = xv(i, e);
    float m = fabsf(xr[0]);
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, fabsf(xr[e]));
    const float s = row16_max(m) / kE4M3Max;
    *reinterpret_cast<uint2 *>(xq + base + (r0 + 16 * i) * K) = quant8f<true>(xr, GroupDiv(s));
    if (sub == 0) sa[kb * M + mb * 128 + r0 + 16 * i] = s;
  }

  // Column tiles (128 tokens of one channel).
  fence_values();
  float cm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float m = fabsf(xv(0, e));
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(xv(i, e)));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    cm[e] = m;
  }
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) colmax[wave][sub * 8 + e] = cm[e];
  }
  __syncthreads();
  if (tid < 128) {
    const float a = fmaxf(fmaxf(colmax[0][tid], colmax[1][tid]), fmaxf(colmax[2][tid], colmax[3][tid]));
    const float s = a / kE4M3Max;
    const GroupDiv d(s);
    colscale[tid] = s;
    colrcp[tid] = d.r;
    colmode[tid] = d.mode;
    sat[mb * K + kb * 128 + tid] = s;
  }
  __syncthreads();
  fence_values();
  float cs[8], cr[8];
  bool all_fast = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    cs[e] = colscale[sub * 8 + e];
    cr[e] = colrcp[sub * 8 + e];
    all_fast = all_fast && colmode[sub * 8 + e] == 1;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (all_fast) {
        GroupDiv d(0.0f);
        d.s = cs[e];
        d.r = cr[e];
        y[e] = d.fast_bf16(xv(i, e));
      } else {
        y[e] = div_any(xv(i, e), cs[e], cr[e], colmode[sub * 8 + e]);
      }
    }
    uint2 q;
    q.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
    q.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2 *>(tile + (r0 + 16 * i) * 32 + sub * 2) = q;
  }
  __syncthreads();
  store_transposed_tile(tile, xqt + (kb * 128) * M + mb * 128, M, tid);
}

hipError_t launch_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sa,
                                 uint8_t *xqt, float *sat, hipStream_t stream) {
  const int64_t blocks = (M / 128) * (K / 128);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_act_dual_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, x, M, K,
                     xq, sa, xqt, sat);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// SwiGLU + 1x128 activation quantizer (the MoE expert down-projection's input): reads the
// up-projection output gu[M][2I] (g = columns 0..I-1, u = I..2I-1) once and writes the
// E4M3 codes of h = SiLU(g) * u, h formed in FP32 (no BF16 round trip), with one online
// scale per 1x128 tile of h.  Same slab layout as the activation quantizer: one wave
// handles 4*NR rows x NK tiles, a tile is one 16-lane DPP row, 16 bytes of g and 16 of u
// per lane.  SiLU(g) = g * sigma(g), sigma from e^-|g| (the library exponential, about one
// ulp; no overflow for any g) and the hardware reciprocal (one ulp).  Values of h below the
// FP32 normal range (|h| < 2^-126) carry the subnormal rounding of the intermediate products.
// ---------------------------------------------------------------------------------------
template <int NR, int NK>
__global__ __launch_bounds__(256) void swiglu_quant_act_1x128_kernel(const uint16_t *__restrict__ gu,
                                                                     int64_t M, int64_t I,
                                                                     uint8_t *__restrict__ xq,
                                                                     float *__restrict__ sa) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kActWavesPerBlock + (threadIdx.x >> 6);
  const int64_t KB = I >> 7;
  const int64_t KG = (KB + NK - 1) / NK;
  const int64_t kb0 = (wave % KG) * NK;
  const int64_t row0 = (wave / KG) * (4 * NR);
  if (row0 >= M) return;
  const int grp = lane >> 4;
  const int sub = lane & 15;
  const int64_t ld = 2 * I;

  uint4 vg[NK][NR], vu[NK][NR];
#pragma unroll
  for (int k = 0; k < NK; ++k)
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t row = row0 + 4 * i + grp;
      const int64_t col = (kb0 + k) * 128 + sub * 8;
      if (row < M && kb0 + k < KB) {
        vg[k][i] = load16_stream(gu + row * ld + col);
        vu[k][i] = load16_stream(gu + row * ld + I + col);
      } else {
        vg[k][i] = make_uint4(0u, 0u, 0u, 0u);
        vu[k][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    if (kb0 + k >= KB) break;
    const int64_t col = (kb0 + k) * 128 + sub * 8;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const uint32_t gw[4] = {vg[k][i].x, vg[k][i].y, vg[k][i].z, vg[k][i].w};
      const uint32_t uw[4] = {vu[k][i].x, vu[k][i].y, vu[k][i].z, vu[k][i].w};
      float h[8];
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = (e & 1) ? bf16_hi(gw[e >> 1]) : bf16_lo(gw[e >> 1]);
        const float u = (e & 1) ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
        // sigma(g) = 1 / (1 + e^-g) for g >= 0 and e^g / (1 + e^g) for g < 0: e^-|g| never
        // overflows
        const float t = expf(-fabsf(g));
        h[e] = g * u * ((g >= 0.0f ? 1.0f : t) * __builtin_amdgcn_rcpf(1.0f + t));
        m = fmaxf(m, fabsf(h[e]));
      }
      const float s = row16_max(m) / kE4M3Max;
      const int64_t row = row0 + 4 * i + grp;
      const uint2 q = quant8f<false>(h, GroupDiv(s));
      if (row < M) *reinterpret_cast<uint2 *>(xq + row * I + col) = q;
      if (sub == 0 && row < M) sa[(kb0 + k) * M + row] = s;
    }
  }
}

hipError_t launch_swiglu_quant_act(const uint16_t *gu, int64_t M, int64_t I, uint8_t *xq, float *sa,
                                   hipStream_t stream) {
  constexpr int NR = 2, NK = 2;
  const int64_t KB = I / 128;
  const int64_t waves = ((M + 4 * NR - 1) / (4 * NR)) * ((KB + NK - 1) / NK);
  const int64_t blocks = (waves + kActWavesPerBlock - 1) / kActWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((swiglu_quant_act_1x128_kernel<NR, NK>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     stream, gu, M, I, xq, sa);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Tensor-level and delayed scaling (the prior art, for accuracy comparisons): one scale for
// a whole tensor of n BF16 values.  stats[0] = amax (float bits; a non-negative float's bits
// order like unsigned integers, so an unsigned atomic max works), stats[1] = saturated
// count, stats[2] = the scale used.  Three launches for tensor-level scaling (clear, amax,
// quantize with amax / 448), two for delayed scaling (clear, quantize with the caller's
// scale while taking the amax for the history).  Grid-stride loops over 16-byte chunks.
// ---------------------------------------------------------------------------------------
__global__ void tensor_stats_clear_kernel(uint32_t *__restrict__ stats) {
  if (threadIdx.x < 3) stats[threadIdx.x] = 0u;
}

// Largest |x| of the workgroup's values, one unsigned atomic max per workgroup.
__device__ __forceinline__ void block_amax_atomic(float m, uint32_t *stats) {
  __shared__ float wmax[4];
  m = row16_max(m);
  m = fmaxf(fmaxf(lane_f32(m, 0), lane_f32(m, 16)), fmaxf(lane_f32(m, 32), lane_f32(m, 48)));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(stats, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

__global__ __launch_bounds__(256) void tensor_amax_kernel(const uint16_t *__restrict__ x, int64_t chunks,
                                                          uint32_t *__restrict__ stats) {
  float m = 0.0f;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * 256)
    m = fmaxf(m, absmax8(load16_stream(x + c * 8)));
  block_amax_atomic(m, stats);
}

// kDelayed: scale from *scale_in (and the amax of x is taken for the history); else from
// the amax already in stats[0].
template <bool kDelayed>
__global__ __launch_bounds__(256) void tensor_quant_kernel(const uint16_t *__restrict__ x, int64_t chunks,
                                                           const float *__restrict__ scale_in,
                                                           uint8_t *__restrict__ q, uint32_t *__restrict__ stats) {
  const float s = kDelayed ? *scale_in : __uint_as_float(stats[0]) / kE4M3Max;
  const GroupDiv dv(s);
  // A caller's scale can put |x/s| beyond the FP32 range; every quotient above 448 maps to
  // the same saturated code, so dividends are clamped to +-512 s first (exact for a mode-1
  // s), which keeps the fast quotient finite and makes the clamped ones exactly +-512.
  const float lim = 512.0f * s;
  float m = 0.0f;
  uint32_t sat = 0;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const uint4 v = load16_stream(x + c * 8);
    float y[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    if (kDelayed) m = fmaxf(m, absmax8(v));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = dv.mode == 1 ? dv.fast_bf16(__builtin_amdgcn_fmed3f(y[i], -lim, lim))
                          : (dv.mode == 2 ? y[i] / dv.s : y[i]);
      sat += fabsf(y[i]) > kE4M3Max ? 1u : 0u;
    }
    uint2 out;
    out.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
    out.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2 *>(q + c * 8) = out;
  }
  if (sat) atomicAdd(stats + 1, sat);
  if (blockIdx.x == 0 && threadIdx.x == 0) stats[2] = __float_as_uint(s);
  if (kDelayed) block_amax_atomic(m, stats);
}

hipError_t launch_quant_per_tensor(const uint16_t *x, int64_t n, const float *scale_in, uint8_t *q,
                                   uint32_t *stats, hipStream_t stream) {
  const int64_t chunks = n / 8;
  const int64_t blocks = (chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096;
  hipLaunchKernelGGL(tensor_stats_clear_kernel, dim3(1), dim3(64), 0, stream, stats);
  if (chunks == 0) return hipGetLastError();
  if (scale_in == nullptr) {
    hipLaunchKernelGGL(tensor_amax_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, x, chunks,
                       stats);
    hipLaunchKernelGGL(tensor_quant_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, x,
                       chunks, scale_in, q, stats);
  } else {
    hipLaunchKernelGGL(tensor_quant_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, x,
                       chunks, scale_in, q, stats);
  }
  return hipGetLastError();
}

}  // namespace fp8q

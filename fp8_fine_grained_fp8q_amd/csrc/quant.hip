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

template <int NR, int NK>
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(const uint16_t *__restrict__ x,
                                                              int64_t M, int64_t K,
                                                              uint8_t *__restrict__ xq,
                                                              float *__restrict__ sa) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kActWavesPerBlock + (threadIdx.x >> 6);
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

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sa,
                            hipStream_t stream) {
  constexpr int NR = FP8Q_ACT_NR, NK = FP8Q_ACT_NK;
  const int64_t KB = K / 128;
  const int64_t waves = ((M + 4 * NR - 1) / (4 * NR)) * ((KB + NK - 1) / NK);
  const int64_t blocks = (waves + kActWavesPerBlock - 1) / kActWavesPerBlock;
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
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(const uint16_t *__restrict__ w,
                                                              int64_t N, int64_t K,
                                                              uint8_t *__restrict__ wq,
                                                              float *__restrict__ sb) {
  __shared__ float wave_max[4];
  const int64_t KB = K >> 7, NB = N >> 7;
  const int64_t bid = blockIdx.x;
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
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2 *>(wq + base + (r0 + 16 * i) * K) = quant8(v[i], dv);
  if (tid == 0) sb[gnb * KB + kb] = s;
  (void)NB;
}

hipError_t launch_quant_w(const uint16_t *w, int64_t G, int64_t N, int64_t K, uint8_t *wq, float *sb,
                          hipStream_t stream) {
  const int64_t blocks = G * (N / 128) * (K / 128);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_w_128x128_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     stream, w, N, K, wq, sb);
  return hipGetLastError();
}

}  // namespace fp8q

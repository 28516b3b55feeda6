// Internal launchers of libfp8q (host side).  Arguments are validated by the C ABI layer
// before any of these is called; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sa,
                            hipStream_t stream);

// launch_quant_act and launch_quant_w (no W^T) for X[M][K] and W[G][N][K] in one launch.
hipError_t launch_quant_act_w(const uint16_t *x, int64_t M, uint8_t *xq, float *sa, const uint16_t *w, int64_t G,
                              int64_t N, uint8_t *wq, float *sb, int64_t K, hipStream_t stream);

// wqt / sbt (W^T codes and block scales) are written too unless wqt is null.
hipError_t launch_quant_w(const uint16_t *w, int64_t G, int64_t N, int64_t K, uint8_t *wq, float *sb,
                          uint8_t *wqt, float *sbt, hipStream_t stream);

// Both orientations of X[M][K] (M % 128 == 0): 1x128 tiles along K (xq, sa as above)
// and 128x1 tiles along M, codes channel-major xqt[K][M], scales sat[M/128][K].
hipError_t launch_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sa,
                                 uint8_t *xqt, float *sat, hipStream_t stream);

// h = SiLU(g) * u of gu[M][2I] (g left half, u right half), quantized in 1x128 tiles.
hipError_t launch_swiglu_quant_act(const uint16_t *gu, int64_t M, int64_t I, uint8_t *xq, float *sa,
                                   hipStream_t stream);

// One scale for n BF16 values (n % 8 == 0): from the tensor's amax (scale_in null) or the
// caller's scale; stats[0..2] = amax bits, saturated count, scale bits.
hipError_t launch_quant_per_tensor(const uint16_t *x, int64_t n, const float *scale_in, uint8_t *q,
                                   uint32_t *stats, hipStream_t stream);

hipError_t launch_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                       int64_t M, int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream);

// C = dequant(aq, sa) dequant(bq, sb)^T, both with 1x128 row scales ([K/128][rows]).
hipError_t launch_gemm_rowscaled(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb,
                                 int64_t M, int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream);

// Debug check of grouped-GEMM offsets (offsets[0] == 0, non-decreasing, offsets[G] == M_tot)
// on `stream`; waits for the stream and sets *bad.
hipError_t check_grouped_offsets(const int32_t *offsets, int64_t G, int64_t M_tot, hipStream_t stream, bool *bad);

hipError_t launch_grouped_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                               const int32_t *offsets, int64_t G, int64_t M_tot, int64_t N, int64_t K,
                               void *c, bool out_f32, hipStream_t stream);

// Expert-parallel dispatch on the GPU owning experts [e_begin, e_begin + E): route the
// top-k ids [T][k] (offsets [E+1], token_row [T][k], row_token [cap]) and pack the routed
// rows' codes xq [T][K] / scales sa [K/128][T] into xq_s [cap][K] / sa_s [K/128][cap].
hipError_t launch_moe_dispatch(const int32_t *ids, int64_t T, int64_t k, int64_t e_begin, int64_t E,
                               const uint8_t *xq, const float *sa, int64_t K, int64_t cap, uint8_t *xq_s,
                               float *sa_s, int32_t *offsets, int32_t *token_row, int32_t *row_token,
                               hipStream_t stream);

// y[t] = sum over slots s with 0 <= token_row[t][s] < cap of w[t][s] * out[token_row[t][s]].
hipError_t launch_moe_combine(const void *out, bool in_f32, int64_t cap, int64_t N, const int32_t *token_row,
                              const float *w, int64_t T, int64_t k, void *y, bool out_f32, hipStream_t stream);

}  // namespace fp8q

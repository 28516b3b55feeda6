// Internal launchers of libfp8q (host side).  Arguments are validated by the C ABI layer
// before any of these is called; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sa,
                            hipStream_t stream);

hipError_t launch_quant_w(const uint16_t *w, int64_t G, int64_t N, int64_t K, uint8_t *wq, float *sb,
                          hipStream_t stream);

hipError_t launch_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                       int64_t M, int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                               const int32_t *offsets, int64_t G, int64_t M_tot, int64_t N, int64_t K,
                               void *c, bool out_f32, hipStream_t stream);

}  // namespace fp8q

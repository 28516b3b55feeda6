// C ABI of libfp8q (see include/fp8q.h): argument checks, then the call's kernel launches.
// Every check runs before the first HIP call, so a bad call never touches the device.
#include "fp8q.h"

#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <mutex>

#include "fp8q_launch.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 62;
constexpr int64_t kMaxGemmK = int64_t(1) << 22;

bool misaligned(const void *p, uintptr_t a = 16) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

bool bad_dim(int64_t v) { return v < 0 || v >= kMaxDim; }

bool too_many(int64_t a, int64_t b) { return a != 0 && b > kMaxElems / a; }

fp8q_status device_ok() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? FP8Q_OK : FP8Q_ERR_DEVICE;
}

fp8q_status launched(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_LAUNCH; }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// FP8Q_DEBUG set to anything but "" or "0" turns on the synchronizing argument checks.
bool debug_checks() {
  const char *v = getenv("FP8Q_DEBUG");
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

// Shared checks of the two GEMM entry points (everything except the grouped extras).
fp8q_status check_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                       int64_t M, int64_t N, int64_t K, void *c, int32_t out_dtype) {
  if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_DTYPE;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8Q_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || N % 128 != 0) return FP8Q_ERR_SHAPE;
  // The kernels address a stage of up to 512 operand rows with 32-bit buffer offsets
  // (row * K + byte), so K is limited to 2^22.
  if (K > kMaxGemmK) return FP8Q_ERR_SHAPE;
  if (too_many(M, K) || too_many(N, K) || too_many(M, N)) return FP8Q_ERR_SHAPE;
  if (M == 0 || N == 0) return 1;  // nothing to do (positive: caller returns FP8Q_OK)
  if (!xq || !sa || !wq || !sb || !c) return FP8Q_ERR_NULL;
  if (misaligned(xq) || misaligned(sa) || misaligned(wq) || misaligned(sb) || misaligned(c))
    return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}

}  // namespace

extern "C" {

fp8q_status fp8q_quantize_act_1x128(const uint16_t *x_bf16, int64_t M, int64_t K, uint8_t *xq,
                                    float *sa, void *stream) {
  if (bad_dim(M) || bad_dim(K) || K % 128 != 0 || too_many(M, K)) return FP8Q_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8Q_OK;
  if (!x_bf16 || !xq || !sa) return FP8Q_ERR_NULL;
  if (misaligned(x_bf16) || misaligned(xq) || misaligned(sa)) return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_quant_act(x_bf16, M, K, xq, sa, as_stream(stream)));
}

fp8q_status fp8q_quantize_w_128x128(const uint16_t *w_bf16, int64_t G, int64_t N, int64_t K,
                                    uint8_t *wq, float *sb, void *stream) {
  if (G < 1 || bad_dim(G) || bad_dim(N) || bad_dim(K)) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (too_many(G, N) || too_many(G * N, K)) return FP8Q_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (!w_bf16 || !wq || !sb) return FP8Q_ERR_NULL;
  if (misaligned(w_bf16) || misaligned(wq) || misaligned(sb)) return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_quant_w(w_bf16, G, N, K, wq, sb, nullptr, nullptr, as_stream(stream)));
}

fp8q_status fp8q_gemm_blockscaled(const uint8_t *xq, const float *sa, const uint8_t *wq,
                                  const float *sb, int64_t M, int64_t N, int64_t K, void *c,
                                  int32_t out_dtype, void *stream) {
  const fp8q_status st = check_gemm(xq, sa, wq, sb, M, N, K, c, out_dtype);
  if (st != FP8Q_OK) return st > 0 ? FP8Q_OK : st;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_gemm(xq, sa, wq, sb, M, N, K, c, out_dtype == FP8Q_OUT_F32,
                                    as_stream(stream)));
}

fp8q_status fp8q_grouped_gemm_blockscaled(const uint8_t *xq, const float *sa, const uint8_t *wq,
                                          const float *sb, const int32_t *offsets, int64_t G,
                                          int64_t M_tot, int64_t N, int64_t K, void *c,
                                          int32_t out_dtype, void *stream) {
  if (G < 1 || bad_dim(G)) return FP8Q_ERR_SHAPE;
  const fp8q_status st = check_gemm(xq, sa, wq, sb, M_tot, N, K, c, out_dtype);
  if (st < 0) return st;
  if (too_many(G, N) || too_many(G * N, K)) return FP8Q_ERR_SHAPE;
  if (st > 0) return FP8Q_OK;
  if (!offsets) return FP8Q_ERR_NULL;
  if (misaligned(offsets, 4)) return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  if (debug_checks()) {
    // One device flag serves the check: checks from several threads run one at a time.
    static std::mutex check_mutex;
    std::lock_guard<std::mutex> lock(check_mutex);
    bool bad = false;
    if (fp8q::check_grouped_offsets(offsets, G, M_tot, as_stream(stream), &bad) != hipSuccess)
      return FP8Q_ERR_LAUNCH;
    if (bad) return FP8Q_ERR_OFFSETS;
  }
  return launched(fp8q::launch_grouped_gemm(xq, sa, wq, sb, offsets, G, M_tot, N, K, c,
                                            out_dtype == FP8Q_OUT_F32, as_stream(stream)));
}

fp8q_status fp8q_quantize_act_w(const uint16_t *x_bf16, int64_t M, const uint16_t *w_bf16, int64_t G, int64_t N,
                                int64_t K, uint8_t *xq, float *sa, uint8_t *wq, float *sb, void *stream) {
  if (bad_dim(M) || bad_dim(K) || K % 128 != 0 || too_many(M, K)) return FP8Q_ERR_SHAPE;
  if (G < 1 || bad_dim(G) || bad_dim(N) || N % 128 != 0) return FP8Q_ERR_SHAPE;
  if (too_many(G, N) || too_many(G * N, K)) return FP8Q_ERR_SHAPE;
  const bool act = M > 0 && K > 0, wts = N > 0 && K > 0;
  if (!act && !wts) return FP8Q_OK;
  if (act && (!x_bf16 || !xq || !sa)) return FP8Q_ERR_NULL;
  if (wts && (!w_bf16 || !wq || !sb)) return FP8Q_ERR_NULL;
  if (act && (misaligned(x_bf16) || misaligned(xq) || misaligned(sa))) return FP8Q_ERR_ALIGN;
  if (wts && (misaligned(w_bf16) || misaligned(wq) || misaligned(sb))) return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_quant_act_w(x_bf16, act ? M : 0, xq, sa, w_bf16, G, wts ? N : 0, wq, sb, K,
                                           as_stream(stream)));
}

fp8q_status fp8q_quantize_w_128x128_t(const uint16_t *w_bf16, int64_t G, int64_t N, int64_t K,
                                      uint8_t *wq, float *sb, uint8_t *wqt, float *sbt, void *stream) {
  if (G < 1 || bad_dim(G) || bad_dim(N) || bad_dim(K)) return FP8Q_ERR_SHAPE;
  if (N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (too_many(G, N) || too_many(G * N, K)) return FP8Q_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (!w_bf16 || !wq || !sb || !wqt || !sbt) return FP8Q_ERR_NULL;
  if (misaligned(w_bf16) || misaligned(wq) || misaligned(sb) || misaligned(wqt) || misaligned(sbt))
    return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_quant_w(w_bf16, G, N, K, wq, sb, wqt, sbt, as_stream(stream)));
}

fp8q_status fp8q_quantize_act_dual(const uint16_t *x_bf16, int64_t M, int64_t K, uint8_t *xq,
                                   float *sa, uint8_t *xqt, float *sat, void *stream) {
  if (bad_dim(M) || bad_dim(K) || M % 128 != 0 || K % 128 != 0 || too_many(M, K)) return FP8Q_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8Q_OK;
  if (!x_bf16 || !xq || !sa || !xqt || !sat) return FP8Q_ERR_NULL;
  if (misaligned(x_bf16) || misaligned(xq) || misaligned(sa) || misaligned(xqt) || misaligned(sat))
    return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_quant_act_dual(x_bf16, M, K, xq, sa, xqt, sat, as_stream(stream)));
}

fp8q_status fp8q_gemm_rowscaled(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb,
                                int64_t P, int64_t Q, int64_t Kc, void *c, int32_t out_dtype,
                                void *stream) {
  const fp8q_status st = check_gemm(aq, sa, bq, sb, P, Q, Kc, c, out_dtype);
  if (st < 0) return st;
  if ((Kc / 128) * Q >= (int64_t(1) << 29)) return FP8Q_ERR_SHAPE;  // scale offsets fit 31 bits
  if (st > 0) return FP8Q_OK;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_gemm_rowscaled(aq, sa, bq, sb, P, Q, Kc, c, out_dtype == FP8Q_OUT_F32,
                                              as_stream(stream)));
}

fp8q_status fp8q_swiglu_quantize_act_1x128(const uint16_t *gu_bf16, int64_t M, int64_t I, uint8_t *xq,
                                           float *sa, void *stream) {
  if (bad_dim(M) || bad_dim(I) || I % 128 != 0 || too_many(M, 2 * I)) return FP8Q_ERR_SHAPE;
  if (M == 0 || I == 0) return FP8Q_OK;
  if (!gu_bf16 || !xq || !sa) return FP8Q_ERR_NULL;
  if (misaligned(gu_bf16) || misaligned(xq) || misaligned(sa)) return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_swiglu_quant_act(gu_bf16, M, I, xq, sa, as_stream(stream)));
}

fp8q_status fp8q_quantize_per_tensor(const uint16_t *x_bf16, int64_t n, const float *scale_in, uint8_t *q,
                                     uint32_t *stats, void *stream) {
  if (n < 0 || n % 8 != 0 || n >= kMaxElems) return FP8Q_ERR_SHAPE;
  if (!stats) return FP8Q_ERR_NULL;
  if (n > 0 && (!x_bf16 || !q)) return FP8Q_ERR_NULL;
  if (misaligned(x_bf16) || misaligned(q) || misaligned(stats, 4) || misaligned(scale_in, 4))
    return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_quant_per_tensor(x_bf16, n, scale_in, q, stats, as_stream(stream)));
}

fp8q_status fp8q_moe_dispatch(const int32_t *topk_ids, int64_t T, int64_t k, int64_t e_begin, int64_t E,
                              const uint8_t *xq, const float *sa, int64_t K, int64_t capacity, uint8_t *xq_sorted,
                              float *sa_sorted, int32_t *offsets, int32_t *token_row, int32_t *row_token,
                              void *stream) {
  if (bad_dim(T) || k < 1 || k > 64 || bad_dim(K) || K % 128 != 0 || E < 1 || E > 1024 || e_begin < 0 ||
      bad_dim(e_begin) || bad_dim(capacity))
    return FP8Q_ERR_SHAPE;
  if (too_many(T, k) || T * k >= kMaxDim || too_many(capacity, K) || too_many(T, K))
    return FP8Q_ERR_SHAPE;
  if (!offsets || (T > 0 && (!topk_ids || !token_row || !xq || !sa)) ||
      (capacity > 0 && (!xq_sorted || !sa_sorted || !row_token)))
    return FP8Q_ERR_NULL;
  if (misaligned(topk_ids, 4) || misaligned(offsets, 4) || misaligned(token_row, 4) || misaligned(row_token, 4) ||
      misaligned(xq) || misaligned(sa) || misaligned(xq_sorted) || misaligned(sa_sorted))
    return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_moe_dispatch(topk_ids, T, k, e_begin, E, xq, sa, K, capacity, xq_sorted, sa_sorted,
                                            offsets, token_row, row_token, as_stream(stream)));
}

fp8q_status fp8q_moe_combine(const void *expert_out, int32_t in_dtype, int64_t capacity, int64_t N,
                             const int32_t *token_row, const float *topk_weights, int64_t T, int64_t k, void *y,
                             int32_t out_dtype, void *stream) {
  if ((in_dtype != FP8Q_OUT_BF16 && in_dtype != FP8Q_OUT_F32) || (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32))
    return FP8Q_ERR_DTYPE;
  if (bad_dim(T) || k < 1 || k > 64 || bad_dim(N) || N % 8 != 0 || bad_dim(capacity) || too_many(T, k) ||
      too_many(capacity, N) || too_many(T, N))
    return FP8Q_ERR_SHAPE;
  if (T == 0 || N == 0) return FP8Q_OK;
  if (!token_row || !topk_weights || !y || (capacity > 0 && !expert_out)) return FP8Q_ERR_NULL;
  if (misaligned(token_row, 4) || misaligned(topk_weights, 4) || misaligned(y) || misaligned(expert_out))
    return FP8Q_ERR_ALIGN;
  if (device_ok() != FP8Q_OK) return FP8Q_ERR_DEVICE;
  return launched(fp8q::launch_moe_combine(expert_out, in_dtype == FP8Q_OUT_F32, capacity, N, token_row,
                                           topk_weights, T, k, y, out_dtype == FP8Q_OUT_F32, as_stream(stream)));
}

const char *fp8q_status_string(fp8q_status status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_NULL: return "null pointer argument";
    case FP8Q_ERR_SHAPE: return "invalid shape (negative, K/N (or M for the dual quantizer) not a multiple of 128, G < 1, or too large)";
    case FP8Q_ERR_ALIGN: return "misaligned pointer (16-byte alignment required; offsets 4-byte)";
    case FP8Q_ERR_DTYPE: return "invalid out_dtype";
    case FP8Q_ERR_DEVICE: return "no usable HIP device";
    case FP8Q_ERR_LAUNCH: return "kernel launch failed";
    case FP8Q_ERR_OFFSETS: return "grouped GEMM offsets invalid (offsets[0] != 0, decreasing, or offsets[G] != M_tot)";
    default: return "unknown status";
  }
}

int32_t fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

}  // extern "C"

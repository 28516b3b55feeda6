/*
 * fp8q.h -- C ABI of libfp8q: online fine-grained FP8 (E4M3) quantization and the
 * block-scaled FP8 GEMM it feeds, for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute, after the DeepSeek-V3 pages:
 *  - dtcms.com DeepSeek-V3 page, section 3 (FP8 mixed-precision training):
 *    3.1 the GEMMs take FP8 tensors and write BF16 or FP32; 3.2 activations are
 *    scaled per 1x128 tile and weights per 128x128 block; 3.3 accumulation
 *    precision is raised by promoting partial sums out of the matrix units.
 *  - codingmall.com page on the role of FP8 precision in DeepSeek-V3 training,
 *    sections "Dinh luong hat min" (fine-grained quantization), "Dinh luong truc
 *    tuyen" (online quantization: every tile's / block's scale comes from its own
 *    current maximum, no history), "Tang do chinh xac tich luy" (partial results
 *    promoted to FP32 registers at fixed K intervals) and "Dinh dang E4M3 hop
 *    nhat" (one format, E4M3, throughout).
 *  - risenshineclean.com DeepSeek training-algorithm page, section 3 (the same
 *    four points; a tile is one token's 128 channels).
 *
 * Numerics shared by every call (readings where the pages are silent):
 *  - E4M3 is the OCP E4M3FN format: bias 7, largest finite 448, S.1111.111 = NaN.
 *  - scale s = RN32(amax / 448) of the tile / block (amax = largest |x|), an FP32
 *    value, not rounded to a power of two; all-zero groups get s = 0;
 *  - code = E4M3(RN32(x / s)), round to nearest even, saturating, sign kept
 *    (-0 -> 0x80); dequantized value = decode(code) * s;  FP32 subnormals kept.
 *  - inputs are finite BF16 (NaN / Inf input: results unspecified).
 *  - GEMM: C[m][n] = sum_kb (sa[kb][m] * sb[n/128][kb]) * P_kb[m][n], where
 *    P_kb = sum over the 128 k of block kb of decode(xq[m][k]) * decode(wq[n][k])
 *    is produced by FP8 matrix-core instructions and each block's P_kb is scaled
 *    and added into an FP32 register accumulator, kb ascending (promotion every
 *    128 K).  C = X * W^T; X is [M][K], W is [N][K], both K-contiguous.
 *
 * Conventions for every entry point:
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA memory) on
 *    the current HIP device; the caller owns all buffers and keeps them alive until
 *    the work on `stream` completes.  Outputs must not alias inputs.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Calls are asynchronous on it and never synchronize the host.  Without FP8Q_DEBUG a
 *    call issues only kernel launches on `stream` (no allocation, memset, copy or wait),
 *    so it can be captured into a HIP graph and replayed; the GEMMs read the CU count
 *    once per device outside any stream, so make one call before capturing.
 *  - Arguments are checked before any HIP call; a failed check returns a negative
 *    fp8q_status and launches nothing.  M == 0 (or M_tot == 0) is a no-op FP8Q_OK.
 *  - Base pointers must be 16-byte aligned.  K and N must be multiples of 128.  The GEMMs
 *    take K (the contraction length) up to 4 194 304 (2^22): their kernels address the
 *    operand stages with 32-bit offsets; larger K returns FP8Q_ERR_SHAPE.
 *  - The library allocates no device memory; its only global state is a per-device
 *    cache of the CU count (written once, the same value by any thread) and the
 *    device flag of the grouped GEMM's offsets check, used only under FP8Q_DEBUG
 *    (the library runs those checks one at a time): calls are reentrant and
 *    thread-safe.  Kernel faults surface at the caller's next synchronization of
 *    `stream`.
 *  - The dense GEMMs pick their kernel and tile plan from the shape and the CU count.
 *    Environment variables override the choice for testing: FP8Q_DENSE_KERNEL ("pp" or
 *    "split"), FP8Q_PP_WIDTH ("256" or "224") and FP8Q_PP_PLAN ("off": no round of
 *    short tiles) for the ping-pong kernel, FP8Q_DENSE_SPLIT ("off", or a count a of
 *    256-wide tile columns) for the split-plan kernel.  Every kernel and plan gives
 *    bit-identical results.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 7

typedef int32_t fp8q_status;

enum {
  FP8Q_OK = 0,
  FP8Q_ERR_NULL = -1,   /* a required pointer is NULL                                   */
  FP8Q_ERR_SHAPE = -2,  /* negative size, K or N not a multiple of 128, G < 1, overflow */
  FP8Q_ERR_ALIGN = -3,  /* a base pointer is not 16-byte aligned                        */
  FP8Q_ERR_DTYPE = -4,  /* out_dtype is neither FP8Q_OUT_BF16 nor FP8Q_OUT_F32          */
  FP8Q_ERR_DEVICE = -5, /* no usable HIP device                                          */
  FP8Q_ERR_LAUNCH = -6,  /* the kernel launch failed (hipGetLastError)                  */
  FP8Q_ERR_OFFSETS = -7  /* grouped GEMM offsets invalid (checked only under FP8Q_DEBUG) */
};

enum { FP8Q_OUT_BF16 = 0, FP8Q_OUT_F32 = 1 };

/*
 * Activation quantizer, one scale per 1x128 tile (one row, 128 consecutive K).
 * Source: codingmall.com FP8-in-DeepSeek-V3 page, sections "Dinh luong hat min" and
 * "Dinh luong truc tuyen"; risenshineclean.com page, section 3 (1x128 tile = one
 * token's 128 channels, scale computed online).
 *   x_bf16 : [M][K] BF16 bit patterns, row-major (row stride K elements)
 *   xq     : [M][K] E4M3 codes (out)
 *   sa     : [K/128][M] FP32 scales (out); sa[kb][m] is the scale of row m, K block kb
 * Requires K % 128 == 0, M >= 0.
 */
fp8q_status fp8q_quantize_act_1x128(const uint16_t *x_bf16, int64_t M, int64_t K, uint8_t *xq,
                                    float *sa, void *stream);

/*
 * Weight quantizer, one scale per 128x128 block, for G stacked matrices.
 * Source: as above (128x128 weight blocks, each scaled independently and online).
 *   w_bf16 : [G][N][K] BF16 bit patterns, row-major
 *   wq     : [G][N][K] E4M3 codes (out)
 *   sb     : [G][N/128][K/128] FP32 scales (out)
 * Requires G >= 1, N % 128 == 0, K % 128 == 0.  N == 0 is a no-op.
 */
fp8q_status fp8q_quantize_w_128x128(const uint16_t *w_bf16, int64_t G, int64_t N, int64_t K,
                                    uint8_t *wq, float *sb, void *stream);

/*
 * Dense block-scaled FP8 GEMM: C = dequant(xq, sa) * dequant(wq, sb)^T.
 * Source: dtcms.com DeepSeek-V3 page, sections 3.1 (FP8 in, BF16/FP32 out) and 3.3;
 * codingmall.com page, section "Tang do chinh xac tich luy" (FP32 promotion at fixed
 * K intervals; here every 128-wide K block, where the scales change).
 *   xq [M][K] codes, sa [K/128][M] FP32  (as written by fp8q_quantize_act_1x128)
 *   wq [N][K] codes, sb [N/128][K/128] FP32 (as written by fp8q_quantize_w_128x128, G=1)
 *   c  [M][N] row-major, BF16 (round to nearest even) or FP32 per out_dtype (out)
 * Requires N % 128 == 0, K % 128 == 0, K >= 128, M >= 0.
 */
fp8q_status fp8q_gemm_blockscaled(const uint8_t *xq, const float *sa, const uint8_t *wq,
                                  const float *sb, int64_t M, int64_t N, int64_t K, void *c,
                                  int32_t out_dtype, void *stream);

/*
 * Grouped (MoE expert) block-scaled FP8 GEMM.  Rows offsets[g] .. offsets[g+1]-1 of the
 * expert-sorted activations are multiplied by expert g's weights:
 *   C[r] = dequant(xq[r], sa[:, r]) * dequant(wq[g], sb[g])^T   for r in expert g's range.
 * Source: as for the dense GEMM; the expert FFN GEMMs of DeepSeekMoE (8 of 256 routed
 * experts active per token: risenshineclean.com page, section 2).
 *   xq [M_tot][K], sa [K/128][M_tot], wq [G][N][K], sb [G][N/128][K/128]
 *   offsets : DEVICE int32 [G+1]; must satisfy offsets[0] == 0, non-decreasing,
 *             offsets[G] == M_tot.  Not checked by default (that needs a sync); the
 *             kernel clamps every range to [0, M_tot).  With the environment variable
 *             FP8Q_DEBUG set (to anything but "" or "0"; read on every call) the call
 *             first checks them on the device, waits for `stream`, and returns
 *             FP8Q_ERR_OFFSETS without launching the GEMM if they are invalid.  The check
 *             uses one flag per device: debug calls on one GPU must not run concurrently
 *             from several host threads.
 *   c [M_tot][N] (out); rows outside every expert range are left untouched.
 * Requires G >= 1, N % 128 == 0, K % 128 == 0, K >= 128, M_tot >= 0.
 */
fp8q_status fp8q_grouped_gemm_blockscaled(const uint8_t *xq, const float *sa, const uint8_t *wq,
                                          const float *sb, const int32_t *offsets, int64_t G,
                                          int64_t M_tot, int64_t N, int64_t K, void *c,
                                          int32_t out_dtype, void *stream);

/*
 * Both online quantizers of a linear layer Y = X W^T in one launch: exactly
 * fp8q_quantize_act_1x128(x_bf16, M, K, xq, sa) and fp8q_quantize_w_128x128(w_bf16, G, N, K,
 * wq, sb) (same sources, same bit-exact outputs), with one kernel boundary instead of two.
 *   x_bf16 [M][K] -> xq [M][K], sa [K/128][M];  w_bf16 [G][N][K] -> wq, sb [G][N/128][K/128]
 * Either part may be empty (M == 0, or N == 0); its pointers are then not used.
 * Errors: FP8Q_ERR_SHAPE (K or N not a multiple of 128, G < 1, overflow), FP8Q_ERR_NULL,
 * FP8Q_ERR_ALIGN (all six pointers 16-byte), FP8Q_ERR_DEVICE, FP8Q_ERR_LAUNCH.
 */
fp8q_status fp8q_quantize_act_w(const uint16_t *x_bf16, int64_t M, const uint16_t *w_bf16, int64_t G, int64_t N,
                                int64_t K, uint8_t *xq, float *sa, uint8_t *wq, float *sb, void *stream);

/*
 * Backward pass of a linear layer Y = X W^T in the same E4M3 format.  Source: the
 * codingmall.com page, section "Dinh dang E4M3 hop nhat", and the risenshineclean.com
 * page, section 3, bullet on the unified E4M3 format (one FP8 format for the forward and
 * the backward pass, made possible by the fine-grained groups); online scales as above.
 * The pages give no formula for the backward GEMMs; these calls follow the plainest
 * reading:
 *  - dgrad dX = dY W: dY is quantized like any activation (fp8q_quantize_act_1x128, tiles
 *    of 128 along N) and W keeps its forward 128x128 blocks, used transposed.  With the
 *    W^T codes and scales from fp8q_quantize_w_128x128_t, dX is fp8q_gemm_blockscaled(dYq,
 *    sa_dY, wqt, sbt, M, K, N, dX, ...).
 *  - wgrad dW = dY^T X: the contraction runs over the tokens, so both operands are
 *    quantized in tiles of 128 consecutive tokens of one channel (fp8q_quantize_act_dual)
 *    and multiplied by fp8q_gemm_rowscaled(dYq^T, s_dY, Xq^T, s_X, N, K, M, dW, ...).
 */

/*
 * Weight quantizer that also writes the transposed codes and scales, reading W once:
 *   w_bf16, wq, sb : as in fp8q_quantize_w_128x128
 *   wqt : [G][K][N] E4M3 codes of W^T (out): wqt[g][k][n] = wq[g][n][k]
 *   sbt : [G][K/128][N/128] FP32 scales of W^T (out): sbt[g][kb][nb] = sb[g][nb][kb]
 * Requires G >= 1, N % 128 == 0, K % 128 == 0.  N == 0 or K == 0 is a no-op.
 * Errors: as fp8q_quantize_w_128x128; wqt and sbt are required (FP8Q_ERR_NULL).
 */
fp8q_status fp8q_quantize_w_128x128_t(const uint16_t *w_bf16, int64_t G, int64_t N, int64_t K,
                                      uint8_t *wq, float *sb, uint8_t *wqt, float *sbt, void *stream);

/*
 * Activation quantizer in both orientations, reading X once:
 *   x_bf16 : [M][K] BF16, row-major (M tokens, K channels)
 *   xq, sa : 1x128 tiles along K, exactly as fp8q_quantize_act_1x128 writes them (out)
 *   xqt    : [K][M] E4M3 codes of X^T, tiles of 128 consecutive tokens of one channel (out)
 *   sat    : [M/128][K] FP32 scales of those tiles (out); sat[mb][k] belongs to tokens
 *            128 mb .. 128 mb + 127 of channel k
 * Requires M % 128 == 0 (pad the token dimension with zero rows), K % 128 == 0.
 * M == 0 or K == 0 is a no-op.  Errors: FP8Q_ERR_SHAPE (M or K not a multiple of 128),
 * FP8Q_ERR_NULL, FP8Q_ERR_ALIGN, FP8Q_ERR_DEVICE, FP8Q_ERR_LAUNCH.
 */
fp8q_status fp8q_quantize_act_dual(const uint16_t *x_bf16, int64_t M, int64_t K, uint8_t *xq,
                                   float *sa, uint8_t *xqt, float *sat, void *stream);

/*
 * FP8 GEMM whose operands both carry 1x128 row-tile scales (the weight-gradient GEMM):
 *   C[p][q] = sum_kb sa[kb][p] * sb[kb][q] * sum_{k in block kb} decode(aq[p][k]) decode(bq[q][k])
 * with the same FP32 promotion per 128-wide K block as the block-scaled GEMM.
 *   aq [P][Kc] codes, sa [Kc/128][P] FP32; bq [Q][Kc] codes, sb [Kc/128][Q] FP32
 *   (for dW: aq = dY^T codes, bq = X^T codes, Kc = tokens, both from fp8q_quantize_act_dual)
 *   c [P][Q] row-major, BF16 or FP32 per out_dtype (out)
 * Requires Q % 128 == 0, Kc % 128 == 0, Kc >= 128, P >= 0, and (Kc/128) * Q * 4 < 2^31.
 * Errors: as fp8q_gemm_blockscaled.
 */
fp8q_status fp8q_gemm_rowscaled(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb,
                                int64_t P, int64_t Q, int64_t Kc, void *c, int32_t out_dtype,
                                void *stream);

/*
 * SwiGLU of an expert up-projection output followed by the 1x128 activation quantizer, in
 * one pass (the input of the MoE down-projection GEMM).  Source: the MoE expert FFN
 * (risenshineclean.com page, section 2) and the online 1x128 quantization of every GEMM
 * activation (codingmall.com page, sections "Dinh luong hat min", "Dinh luong truc
 * tuyen").  The pages do not name the activation; SwiGLU h = SiLU(g) * u is the reading.
 *   gu_bf16 : [M][2I] BF16 row-major; g = columns 0..I-1, u = columns I..2I-1
 *   xq      : [M][I] E4M3 codes of h (out), h formed in FP32 from the BF16 g and u
 *   sa      : [I/128][M] FP32 tile scales of h (out)
 * SiLU(g) = g / (1 + e^-g) is computed in FP32 with about two ulps of error, so codes can
 * differ from a correctly rounded h where h / s lies within a few ulps of an E4M3
 * rounding boundary; values of h below the FP32 normal range (|h| < 2^-126, e.g. gates
 * below -87) are not reproduced to that accuracy.  Requires I % 128 == 0, M >= 0.
 * Errors as the activation quantizer.
 */
fp8q_status fp8q_swiglu_quantize_act_1x128(const uint16_t *gu_bf16, int64_t M, int64_t I, uint8_t *xq,
                                           float *sa, void *stream);

/*
 * Tensor-level and delayed FP8 scaling, the prior art the fine-grained online scheme is
 * contrasted with (risenshineclean.com page, section 3, first bullet: 1x128 / 128x128
 * groups versus traditional tensor-level quantization; codingmall.com page, section "Dinh
 * luong truc tuyen": no delayed quantization from historical maxima).  For accuracy
 * comparisons only: one scale for a whole tensor.
 *   x_bf16   : n BF16 values (any layout), n % 8 == 0
 *   scale_in : NULL for tensor-level scaling (scale = RN32(amax / 448) of x itself), or a
 *              DEVICE float holding the scale to use (delayed scaling: the caller forms it
 *              from the amax history, e.g. RN32(max(history) / 448))
 *   q        : n E4M3 codes (out), code = E4M3(RN32(x / scale)), saturating at +-448
 *   stats    : DEVICE uint32[3] (out): [0] = bits of the FP32 amax of x (for the history),
 *              [1] = number of values whose quotient exceeded 448 and saturated,
 *              [2] = bits of the FP32 scale used
 * The codes feed fp8q_gemm_blockscaled with every tile / block scale equal to the tensor's
 * scale.  n == 0 only clears stats.  Errors: FP8Q_ERR_SHAPE (n < 0 or n % 8 != 0),
 * FP8Q_ERR_NULL, FP8Q_ERR_ALIGN (x, q 16-byte; stats, scale_in 4-byte), FP8Q_ERR_DEVICE,
 * FP8Q_ERR_LAUNCH.
 */
fp8q_status fp8q_quantize_per_tensor(const uint16_t *x_bf16, int64_t n, const float *scale_in, uint8_t *q,
                                     uint32_t *stats, void *stream);

/*
 * Expert-parallel dispatch, one GPU's share: the GPU owning experts [e_begin, e_begin + E)
 * lays out the tokens routed to them for the grouped GEMM.  Source: dlbhg.com page on
 * DeepSeek-V3's training techniques, section 1.1 item 2 (8 of 256 routed experts per token),
 * section 2.1 (64-way expert parallelism) and section 3.1 (all-to-all dispatch and combine);
 * dtcms.com page, the DualPipe paragraph (dispatch and combine stages).  The all-to-all
 * exchange itself is not part of this library; this is the work that sends (or, run on the
 * received tokens, receives) E4M3 codes plus 1x128 tile scales, which is what the pages'
 * FP8 scheme makes the payload (the quantizer is row-local, so quantizing before the
 * exchange equals quantizing after it).
 *   topk_ids   : DEVICE int32 [T][k], global expert ids (1 <= k <= 64; ids outside the local
 *                range are skipped)
 *   xq, sa     : the tokens' codes [T][K] and tile scales [K/128][T] (fp8q_quantize_act_1x128)
 *   capacity   : rows of the outputs.  T*k always suffices; with fewer, the rows from
 *                `capacity` on are dropped (their slots get token_row -1) while offsets
 *                still count them, so offsets[E] > capacity tells the caller it was short
 *   xq_sorted  : [capacity][K] out, sa_sorted : [K/128][capacity] out
 *   offsets    : [E+1] out: expert e's rows are offsets[e] .. offsets[e+1]-1, experts in order,
 *                tokens ascending within an expert (the grouped GEMM's offsets, with
 *                M_tot = capacity, which clamps them; rows from offsets[E] on are not written)
 *   token_row  : [T][k] out: the row of (t, s), or -1 if its expert is not local
 *   row_token  : [capacity] out: the token of each row < offsets[E]
 * Requires K % 128 == 0, 1 <= E <= 1024; with T == 0 only `offsets` is written (zeros).
 * Up to four launches (count, scan and rank over chunks of 1024 entries, then the copy);
 * token_row serves as the count pass's scratch.  Errors: FP8Q_ERR_SHAPE, FP8Q_ERR_NULL, FP8Q_ERR_ALIGN (index arrays 4-byte, the
 * rest 16-byte), FP8Q_ERR_DEVICE, FP8Q_ERR_LAUNCH.
 */
fp8q_status fp8q_moe_dispatch(const int32_t *topk_ids, int64_t T, int64_t k, int64_t e_begin, int64_t E,
                              const uint8_t *xq, const float *sa, int64_t K, int64_t capacity, uint8_t *xq_sorted,
                              float *sa_sorted, int32_t *offsets, int32_t *token_row, int32_t *row_token,
                              void *stream);

/*
 * Expert-parallel combine, one GPU's share (sources as for fp8q_moe_dispatch):
 *   y[t][n] = sum over slots s with 0 <= token_row[t][s] < capacity of
 *             topk_weights[t][s] * expert_out[token_row[t][s]][n],
 * FP32 fused multiply-adds in slot order, then y in out_dtype (BF16 round to nearest even,
 * or FP32).  This is the local part of a token's output; the other GPUs' parts add the same
 * way after the combine exchange.
 *   expert_out : [capacity][N] in in_dtype (FP8Q_OUT_BF16 or FP8Q_OUT_F32), e.g. the
 *                grouped GEMM's output on the dispatched rows
 *   token_row, topk_weights : DEVICE [T][k] (fp8q_moe_dispatch; the gating weights)
 *   y : [T][N] out.  Requires N % 8 == 0.  Errors: FP8Q_ERR_DTYPE, FP8Q_ERR_SHAPE,
 *   FP8Q_ERR_NULL, FP8Q_ERR_ALIGN, FP8Q_ERR_DEVICE, FP8Q_ERR_LAUNCH.
 */
fp8q_status fp8q_moe_combine(const void *expert_out, int32_t in_dtype, int64_t capacity, int64_t N,
                             const int32_t *token_row, const float *topk_weights, int64_t T, int64_t k, void *y,
                             int32_t out_dtype, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *fp8q_status_string(fp8q_status status);

/* FP8Q_ABI_VERSION of the built library. */
int32_t fp8q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */

"""Backward-pass FP8 GEMMs of a linear layer in the single E4M3 format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say that one FP8 format, E4M3, serves both the forward and the backward
pass, which the fine-grained grouping makes possible (codingmall.com page on FP8 in
DeepSeek-V3 training, section "Dinh dang E4M3 hop nhat"; risenshineclean.com training-
algorithm page, section 3, bullet "unified E4M3 format"), and that every activation
tile and weight block is scaled online (same pages, "online quantization").  They give no
formula for the backward GEMMs.  Readings, for a layer Y = X W^T with X[M][K],
W[N][K] and the output gradient dY[M][N]:

* dgrad  dX = dY W  (contraction over N).  dY is an activation: it is quantized in
  1x128 tiles along its contraction dimension N by the forward activation quantizer.
  W keeps the 128x128 blocks of the forward pass: block (nb, kb) is used transposed,
  with the same codes and the same scale.  So dgrad is the forward block-scaled GEMM
  with the operands (dYq, sa_dY) and (W^T codes, sb^T).
* wgrad  dW = dY^T X  (contraction over the M tokens).  Both operands are quantized in
  tiles of 128 along the contraction dimension, i.e. 128 consecutive tokens of one
  channel (a 128x1 tile of the token-major layout), each with its own online scale
  amax/448: s_dY[mb][n] and s_X[mb][k].  The codes are stored channel-major (the
  transposes dY^T[N][M], X^T[K][M]) so that the contraction dimension is contiguous,
  and dW[n][k] = sum_mb s_dY[mb][n] s_X[mb][k] sum_{m in mb} dec(dY^T q[n][m]) dec(X^T q[k][m]).
  The token count M is a multiple of 128 here (a caller pads with zero tokens, which
  change neither the sums nor any amax).
* Acceptance as in the forward GEMM: |C_gpu - C| <= 2e-3 ||a_hat_row|| ||b_hat_row||.

Functions are the plain definitions: transposition of codes and scales, the forward
activation quantizer applied to the transposed matrix, and the FP64 product of the
dequantized operands (a library matmul).

Parity status: pinned (the transposed-operand forms equal the direct products of the
dequantized originals; a pure-Python rational brute force of a 128x1 tile quantizer
and of a tiny wgrad; closed forms for constant operands).
"""
from __future__ import annotations

import numpy as np

from . import quant


def transpose_w_blocks(wq: np.ndarray, sb: np.ndarray):
    """Weight codes and block scales of W[.., N, K] -> those of W^T[.., K, N]:
    (wq^T uint8 [G][K][N], sb^T float32 [G][K/128][N/128]) (2-D inputs stay 2-D)."""
    return (np.ascontiguousarray(np.swapaxes(wq, -1, -2)),
            np.ascontiguousarray(np.swapaxes(sb, -1, -2)))


def quantize_act_128x1(x_bf16: np.ndarray):
    """Tiles of 128 consecutive rows (tokens) of one column: x_bf16 uint16 [M][C] with M a
    multiple of 128 -> (codes of x^T uint8 [C][M], scales float32 [M/128][C]).
    This is the 1x128 activation quantizer applied to x^T."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    if x_bf16.shape[0] % quant.TILE:
        raise ValueError("the token count must be a multiple of 128")
    return quant.quantize_act_1x128(np.ascontiguousarray(x_bf16.T))


def dgrad(dyq, sa_dy, wq, sb) -> np.ndarray:
    """dX [M][K] = dequant(dYq) . dequant(W) via the transposed-block operands."""
    wqt, sbt = transpose_w_blocks(wq, sb)
    return quant.dequant_act(dyq, sa_dy) @ quant.dequant_w(wqt, sbt).T


def gemm_rowscaled(aq, sa, bq, sb) -> np.ndarray:
    """A B^T with per-row 1x128 tile scales on both operands: aq uint8 [P][Kc],
    sa float32 [Kc/128][P], bq uint8 [Q][Kc], sb float32 [Kc/128][Q] -> float64 [P][Q]."""
    return quant.dequant_act(aq, sa) @ quant.dequant_act(bq, sb).T


def wgrad(dyq_t, s_dy, xq_t, s_x) -> np.ndarray:
    """dW [N][K] from the channel-major codes of dY^T [N][M] and X^T [K][M]."""
    return gemm_rowscaled(dyq_t, s_dy, xq_t, s_x)


def row_norms_rowscaled(q, s) -> np.ndarray:
    return np.linalg.norm(quant.dequant_act(q, s), axis=1)

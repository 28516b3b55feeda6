"""Block-scaled FP8 GEMM, dense and grouped (MoE experts): the exact dequantized product.

What the method computes (dtcms.com DeepSeek-V3 page, section 3.1: FP8
tensors in, BF16 or FP32 out; section 3.3 and the codingmall.com page on FP8
in DeepSeek-V3 training, section "Tang do chinh xac tich luy": partial sums
are promoted to FP32 registers at fixed K intervals, where the tile and block
scales apply) reaches, up to rounding order, the product of the dequantized
operands

    C[m][n] = sum_k x_hat[m][k] * w_hat[n][k]
            = sum_kb sa[kb][m] * sb[n/128][kb] * sum_{k in kb} dec(xq[m][k]) * dec(wq[n][k]).

This oracle is that definition written out: dequantize both operands exactly
in float64 and multiply them with a float64 matrix product (a library
primitive).  It does not imitate the promotion schedule.  Readings:

* orientation C = X * W^T, X[M][K] and W[N][K] both K-contiguous;
* grouped (MoE) form: rows offsets[g] .. offsets[g+1]-1 of X use expert g's
  weights W[g] and scales sb[g]; rows outside every range are not produced;
* acceptance: |C_gpu - C| <= 2e-3 * ||x_hat[m]||_2 * ||w_hat[n]||_2 per
  element, C_gpu compared as stored (BF16 output rounding counted inside the
  bound), norms of the dequantized operands in float64.

Parity status: pinned (pure-Python exact rational brute force on small shapes,
the blocked integer form, closed forms for constant operands, G=1 and
concatenation reductions for the grouped form).  The GPU's within-block MFMA
summation order is not modelled; the acceptance bound covers it.
"""
from __future__ import annotations

import numpy as np

from . import e4m3, quant

TOL_REL = 2e-3


def gemm_blockscaled(xq, sa, wq, sb) -> np.ndarray:
    """Dense: xq uint8 [M][K], sa f32 [K/128][M], wq uint8 [N][K], sb f32 [N/128][K/128]
    -> C float64 [M][N]."""
    xh = quant.dequant_act(xq, sa)
    wh = quant.dequant_w(wq, sb)
    return xh @ wh.T


def grouped_gemm_blockscaled(xq, sa, wq, sb, offsets) -> np.ndarray:
    """Grouped: xq [M_tot][K], sa [K/128][M_tot], wq [G][N][K], sb [G][N/128][K/128],
    offsets int [G+1] -> C float64 [M_tot][N]; rows in no expert range are NaN."""
    M = xq.shape[0]
    G, N, _ = wq.shape
    out = np.full((M, N), np.nan)
    xh = quant.dequant_act(xq, sa)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            out[lo:hi] = xh[lo:hi] @ quant.dequant_w(wq[g], sb[g]).T
    return out


def gemm_entries(xq, sa, wq, sb, rows, cols) -> np.ndarray:
    """C at selected (row, col) pairs only, for full-size spot checks (dense form):
    each entry is the float64 dot product of one dequantized X row and one
    dequantized W row."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    K = xq.shape[1]
    kb = K // quant.TILE
    xh = {}
    for r in np.unique(rows):
        d = e4m3.decode(xq[r]).reshape(kb, quant.TILE)
        xh[int(r)] = (d * sa[:, r].astype(np.float64)[:, None]).reshape(K)
    wh = {}
    for c in np.unique(cols):
        d = e4m3.decode(wq[c]).reshape(kb, quant.BLOCK)
        wh[int(c)] = (d * sb[c // quant.BLOCK].astype(np.float64)[:, None]).reshape(K)
    out = np.empty(len(rows))
    for i, (r, c) in enumerate(zip(rows, cols)):
        out[i] = float(xh[int(r)] @ wh[int(c)])
    return out


def row_norms_act(xq, sa) -> np.ndarray:
    return np.linalg.norm(quant.dequant_act(xq, sa), axis=1)


def row_norms_w(wq, sb) -> np.ndarray:
    return np.linalg.norm(quant.dequant_w(wq, sb), axis=-1)


def tolerance(xnorm, wnorm) -> np.ndarray:
    """Per-element bound 2e-3 * ||x_hat[m]|| * ||w_hat[n]|| (outer product of the norms)."""
    return TOL_REL * np.outer(np.asarray(xnorm, np.float64), np.asarray(wnorm, np.float64))

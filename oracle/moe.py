"""Expert-parallel dispatch and combine around the grouped GEMM, one GPU's share
(TEST INFRASTRUCTURE ONLY, see the package docstring).

What the pages fix: each token activates 8 of 256 routed experts (dlbhg.com page,
section 1.1, item 2: DeepSeekMoE), experts are spread over the GPUs by 64-way expert
parallelism (same page, section 2.1), and tokens travel to their experts and back with
all-to-all dispatch and combine (same page, section 3.1; dtcms.com page, the DualPipe
paragraph of its section on pipeline parallelism, which names the dispatch and combine
stages of a block).

Readings (the pages give no formula for either step):
* dispatch, on the GPU that owns experts [e_begin, e_begin + E): every (token t, slot s)
  whose routed expert is local becomes one row of the expert-sorted layout the grouped GEMM
  takes: experts in order, and within an expert the tokens in increasing index.  The row
  carries the token's E4M3 codes and its 1x128 tile scales; quantizing before the exchange
  is the same as quantizing after it, because the activation quantizer is row-local.
* combine: y[t] = sum over the token's slots s whose expert is local of w[t, s] * out[row],
  w the gating weight of that slot (an input: the router is not part of this path).  On
  one GPU this is that GPU's part of the sum; the other GPUs' parts come back with the
  combine all-to-all and add up the same way.
Parity status: pinned (brute-force loops, the routing lists the workloads derive from the
same ids, row-locality of the quantizer, closed forms of the combine).
"""
from __future__ import annotations

import numpy as np


def dispatch(topk_ids: np.ndarray, e_begin: int, n_local: int):
    """topk_ids int [T][k] (global expert ids) -> (offsets int32 [E+1], row_token int64 [R],
    token_row int32 [T][k] with -1 for slots whose expert is not local)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    local = ids - e_begin
    is_local = (local >= 0) & (local < n_local)
    counts = np.array([np.count_nonzero(local[is_local] == e) for e in range(n_local)], dtype=np.int64)
    offsets = np.zeros(n_local + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    token_row = np.full((T, k), -1, dtype=np.int32)
    row_token = np.zeros(int(offsets[-1]), dtype=np.int64)
    for e in range(n_local):
        t_idx, s_idx = np.nonzero(is_local & (local == e))  # row-major: tokens ascending
        rows = offsets[e] + np.arange(t_idx.size)
        token_row[t_idx, s_idx] = rows
        row_token[rows] = t_idx
    return offsets, row_token, token_row


def pack(xq: np.ndarray, sa: np.ndarray, row_token: np.ndarray):
    """Rows of the quantized tokens in dispatch order: codes xq[T][K] -> [R][K], scales
    sa[K/128][T] -> [K/128][R]."""
    return xq[row_token], sa[:, row_token]


def combine(out: np.ndarray, token_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """y[t] = sum_s w[t, s] * out[token_row[t, s]] over the local slots, in float64."""
    out = np.asarray(out, dtype=np.float64)
    T, k = token_row.shape
    y = np.zeros((T, out.shape[1]), dtype=np.float64)
    for s in range(k):
        r = token_row[:, s]
        m = r >= 0
        y[m] += np.asarray(weights, dtype=np.float64)[m, s, None] * out[r[m]]
    return y


def combine_bound(out: np.ndarray, token_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """sum_s |w[t, s] * out[row]| per output element: the scale of the combine's rounding."""
    return combine(np.abs(np.asarray(out, dtype=np.float64)), token_row, np.abs(weights))

"""Pins for the oracle's block-scaled GEMM (dense and grouped), CPU only.

Fixed by: exact rational brute force on small shapes (codes decoded by torch's
float8_e4m3fn, not by the oracle's table); the blocked form with exact
integer partial sums per 128-wide K block, which is how the promotion scheme
organises the same sum; closed forms for constant operands; the reductions
G=1 -> dense and grouped -> concatenation of dense per-expert products; and
planted mistakes that the acceptance bound must reject."""
from fractions import Fraction

import numpy as np
import torch

import workloads as wl
from oracle import gemm, quant


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _quantized(M, N, K, seed, G=None):
    rng = np.random.default_rng(seed)
    x = wl.bf16_bits(rng.standard_normal((M, K), dtype=np.float32) * np.float32(2))
    shape = (N, K) if G is None else (G, N, K)
    w = wl.bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02))
    xq, sa = quant.quantize_act_1x128(x)
    wq, sb = quant.quantize_w_128x128(w)
    return xq, sa, wq, sb


def test_dense_matches_exact_rational_brute_force():
    M, N, K = 5, 256, 384
    xq, sa, wq, sb = _quantized(M, N, K, 1)
    C = gemm.gemm_blockscaled(xq, sa, wq, sb)
    assert C.shape == (M, N)
    xd, wd = torch_decode(xq), torch_decode(wq)
    cols = [0, 1, 77, 127, 128, 200, 255]
    for m in range(M):
        for n in cols:
            exact = Fraction(0)
            mag = 0.0
            for k in range(K):
                t = (Fraction(float(xd[m, k])) * Fraction(float(sa[k // 128, m]))
                     * Fraction(float(wd[n, k])) * Fraction(float(sb[n // 128, k // 128])))
                exact += t
                mag += abs(float(t))
            assert abs(C[m, n] - float(exact)) <= 1e-13 * mag + 1e-300, (m, n)


def test_dense_equals_blocked_integer_partials():
    """sum_kb sa*sb * P_kb with P_kb the exact integer sum of (code value * 2^9) products."""
    M, N, K = 33, 384, 640
    xq, sa, wq, sb = _quantized(M, N, K, 2)
    C = gemm.gemm_blockscaled(xq, sa, wq, sb)
    ia = np.rint(torch_decode(xq) * 512).astype(np.int64)
    ib = np.rint(torch_decode(wq) * 512).astype(np.int64)
    assert np.all(np.abs(ia) <= 229376) and np.all(np.abs(ib) <= 229376)
    ref = np.zeros((M, N))
    for kb in range(K // 128):
        P = ia[:, kb * 128:(kb + 1) * 128] @ ib[:, kb * 128:(kb + 1) * 128].T   # exact int64
        scale = sa[kb].astype(np.float64)[:, None] * np.repeat(sb[:, kb], 128).astype(np.float64)[None, :]
        ref += scale * P.astype(np.float64) * 2.0 ** -18
    assert np.allclose(C, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_constant_operands_closed_form():
    M, N, K = 4, 128, 512
    x = wl.bf16_bits(np.full((M, K), 3.0, np.float32))
    w = wl.bf16_bits(np.full((N, K), -0.5, np.float32))
    xq, sa = quant.quantize_act_1x128(x)
    wq, sb = quant.quantize_w_128x128(w)
    C = gemm.gemm_blockscaled(xq, sa, wq, sb)
    want = K * (448.0 * float(np.float32(3.0) / np.float32(448))) * (-448.0 * float(np.float32(0.5) / np.float32(448)))
    assert np.allclose(C, want, rtol=1e-14, atol=0)   # exact terms, FP64 summation


def test_orientation_is_x_times_w_transposed():
    """Non-square, distinct rows: C[m][n] pairs row m of X with row n of W."""
    M, N, K = 2, 128, 128
    x = np.zeros((M, K), np.float32)
    x[0, 0], x[1, 5] = 448.0, 448.0
    w = np.zeros((N, K), np.float32)
    w[7, 0] = 448.0
    w[9, 5] = 224.0
    w[0, 127] = 448.0                                 # sets the block scale to 1
    xq, sa = quant.quantize_act_1x128(wl.bf16_bits(x))
    wq, sb = quant.quantize_w_128x128(wl.bf16_bits(w))
    C = gemm.gemm_blockscaled(xq, sa, wq, sb)
    assert C[0, 7] == 448.0 * 448.0 and C[1, 9] == 448.0 * 224.0
    assert np.count_nonzero(C) == 2


def test_grouped_reductions():
    G, N, K = 3, 256, 256
    offsets = np.array([0, 50, 50, 170], np.int32)    # expert 1 is empty
    xq, sa, wq, sb = _quantized(170, N, K, 3, G=G)
    Cg = gemm.grouped_gemm_blockscaled(xq, sa, wq, sb, offsets)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            Cd = gemm.gemm_blockscaled(xq[lo:hi], np.ascontiguousarray(sa[:, lo:hi]), wq[g], sb[g])
            assert np.array_equal(Cg[lo:hi], Cd)
    one = gemm.grouped_gemm_blockscaled(xq, sa, wq[:1], sb[:1], np.array([0, 170], np.int32))
    assert np.array_equal(one, gemm.gemm_blockscaled(xq, sa, wq[0], sb[0]))
    # rows outside every range are not produced
    part = gemm.grouped_gemm_blockscaled(xq, sa, wq[:1], sb[:1], np.array([0, 100], np.int32))
    assert np.all(np.isnan(part[100:])) and not np.any(np.isnan(part[:100]))


def test_entries_match_full_product():
    xq, sa, wq, sb = _quantized(40, 384, 512, 4)
    C = gemm.gemm_blockscaled(xq, sa, wq, sb)
    rows = [0, 3, 39, 17]
    cols = [383, 0, 128, 255]
    e = gemm.gemm_entries(xq, sa, wq, sb, rows, cols)
    assert np.allclose(e, C[rows, cols], rtol=1e-13, atol=1e-13)


def test_tolerance_accepts_bf16_rounding_and_rejects_planted_mistakes():
    """The acceptance bound must admit the BF16-rounded exact result yet reject the
    mistakes a kernel could plausibly make (a dropped K block, a scale from the wrong
    row, a swapped pair of K blocks' weight scales)."""
    c = wl.tiny()
    xq, sa = quant.quantize_act_1x128(c["x"])
    wq, sb = quant.quantize_w_128x128(c["w"][0])
    C = gemm.gemm_blockscaled(xq, sa, wq, sb)
    tol = gemm.tolerance(gemm.row_norms_act(xq, sa), gemm.row_norms_w(wq, sb))
    bf16 = torch.from_numpy(C.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.all(np.abs(bf16 - C) <= tol)
    # dropped last K block
    drop = gemm.gemm_blockscaled(xq[:, :384], np.ascontiguousarray(sa[:3]), wq[:, :384], np.ascontiguousarray(sb[:, :3]))
    assert np.any(np.abs(drop - C) > tol)
    # activation scale taken from the neighbouring row
    sa_bad = np.ascontiguousarray(np.roll(sa, 1, axis=1))
    assert np.any(np.abs(gemm.gemm_blockscaled(xq, sa_bad, wq, sb) - C) > tol)
    # weight scales of K blocks 0 and 1 swapped
    sb_bad = sb.copy()
    sb_bad[:, [0, 1]] = sb_bad[:, [1, 0]]
    assert np.any(np.abs(gemm.gemm_blockscaled(xq, sa, wq, sb_bad) - C) > tol)

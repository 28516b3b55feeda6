"""The FP32 promotion tripwire: operands on which the matrix core's block sums are exact,
and the a-priori bound on what the FP32 promotion alone may add.

Operands: E4M3 codes of small integers (|value| <= 8), so every product is an integer of
magnitude <= 64 and every 128-wide block sum an integer of magnitude <= 8192, which the
FP8 matrix core sums exactly (products this close in magnitude lose no bits to its
alignment); scales are random FP32 numbers with full 24-bit significands, so that the
promotion, acc = RN(t * P_kb + acc) with t = RN(sa * sb), does real rounding work.

Bound (FP32, u = 2^-24), for promotion in ascending K-block order with one rounding of the
scale product and one rounding per fold (the method's FP32 accumulation at every 128-wide
K interval, codingmall.com page on FP8 in DeepSeek-V3 training, section "Tang do chinh xac
tich luy"):
    acc_kb = (t_kb P_kb + acc_{kb-1})(1 + d_kb),  t_kb = sa sb (1 + e_kb),  |d|, |e| <= u
    |C_gpu - C| <= u * (sum_kb |S_kb| + 2 sum_kb |sa sb P_kb|) * (1 + 2 KB u)
with S_kb = sum_{j <= kb} sa_j sb_j P_j the exact running sums.  The factor 2 also covers
a promotion that multiplies by the two scales one after the other (two roundings).
A regression in the K loop that loses precision -- a scale product or a partial kept in a
narrower format, a partial folded twice or into the wrong block, a different fold order --
breaks it (tests/test_promotion_tripwire.py shows this on emulations, on the CPU).
"""
import numpy as np

from oracle import e4m3

U = 2.0 ** -24


def int_codes(shape, rng):
    """E4M3 codes of uniformly drawn integers in [-8, 8]."""
    v = rng.integers(-8, 9, size=shape).astype(np.float32)
    return e4m3.encode(v)


def full_mantissa_scales(shape, rng, lo=-6, hi=6):
    """Positive FP32 numbers 2^e * (1 + f), e in [lo, hi), f with 23 random bits."""
    m = rng.integers(1 << 23, 1 << 24, size=shape).astype(np.float64)
    e = rng.integers(lo, hi, size=shape)
    return np.ldexp(m, e - 23).astype(np.float32)


def block_partials(aq, bq):
    """P[kb][i][j] = sum over block kb of dec(aq[i,k]) * dec(bq[j,k]) (exact integers)."""
    a = e4m3.decode(aq).astype(np.float64)
    b = e4m3.decode(bq).astype(np.float64)
    KB = a.shape[1] // 128
    return np.stack([a[:, kb * 128:(kb + 1) * 128] @ b[:, kb * 128:(kb + 1) * 128].T for kb in range(KB)])


def exact_and_bound(P, scale):
    """P [KB][M][N] exact block partials, scale [KB][M][N] = sa * sb in float64 (exact).
    Returns (C exact, per-element bound)."""
    terms = scale * P
    run = np.cumsum(terms, axis=0)
    KB = P.shape[0]
    bound = U * (np.abs(run).sum(axis=0) + 2.0 * np.abs(terms).sum(axis=0)) * (1.0 + 2.0 * KB * U)
    return run[-1], bound


def dense_case(M, N, K, seed):
    """(xq, sa [K/128][M], wq, sb [N/128][K/128], C, bound) for C = X W^T."""
    rng = np.random.default_rng(seed)
    xq, wq = int_codes((M, K), rng), int_codes((N, K), rng)
    sa = full_mantissa_scales((K // 128, M), rng)
    sb = full_mantissa_scales((N // 128, K // 128), rng)
    P = block_partials(xq, wq)
    sbn = np.repeat(sb.astype(np.float64), 128, axis=0)          # [N][KB]
    scale = sa.astype(np.float64)[:, :, None] * sbn.T[:, None, :]
    C, bound = exact_and_bound(P, scale)
    return xq, sa, wq, sb, C, bound


def rowscaled_case(M, N, K, seed):
    """Both operands with 1x128 row scales: (aq, sa [K/128][M], bq, sb [K/128][N], C, bound)."""
    rng = np.random.default_rng(seed)
    aq, bq = int_codes((M, K), rng), int_codes((N, K), rng)
    sa = full_mantissa_scales((K // 128, M), rng)
    sb = full_mantissa_scales((K // 128, N), rng)
    P = block_partials(aq, bq)
    scale = sa.astype(np.float64)[:, :, None] * sb.astype(np.float64)[:, None, :]
    C, bound = exact_and_bound(P, scale)
    return aq, sa, bq, sb, C, bound


def check(got, C, bound, what=""):
    """Asserts |got - C| <= bound element-wise; returns the largest error / bound."""
    got = np.asarray(got, np.float64)
    assert got.shape == C.shape, what
    err = np.abs(got - C)
    ratio = err / np.maximum(bound, 1e-300)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bound), (f"{what}: {np.count_nonzero(err > bound)} elements beyond the promotion bound; "
                                  f"worst at {worst}: got {got[worst]!r} exact {C[worst]!r} bound {bound[worst]:.3g}")
    print(f"[{what}] max |err| / promotion bound = {float(ratio.max()):.3f}", flush=True)
    return float(ratio.max())

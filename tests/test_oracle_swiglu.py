"""Pins for the oracle's SwiGLU + 1x128 quantization (CPU only): SiLU's odd-part identity
SiLU(x) - SiLU(-x) = x, the tanh form SiLU(x) = x/2 (1 + tanh(x/2)), printed values of the
logistic function, extreme arguments, the g/u column split (a swapped half fails), and the
composition with the pinned FP32-input quantizer (equal to the BF16 quantizer on values
that are exactly BF16)."""
import math

import numpy as np

import workloads as wl
from oracle import quant, swiglu


def bf16(a):
    return wl.bf16_bits(np.asarray(a, dtype=np.float32))


def gu_of(g, u):
    return np.concatenate([bf16(g), bf16(u)], axis=1)


def test_silu_identities():
    rng = np.random.default_rng(1)
    g = rng.standard_normal((4, 128)) * 6
    gb = quant.bf16_to_f32(bf16(g)).astype(np.float64)
    ones = np.ones_like(g)
    h_pos = swiglu.swiglu_f64(gu_of(g, ones))
    h_neg = swiglu.swiglu_f64(gu_of(-g, ones))
    np.testing.assert_allclose(h_pos - h_neg, gb, rtol=1e-13, atol=4e-15)
    # the tanh form cancels for very negative x, so compare where 1 + tanh(x/2) keeps its bits
    keep = gb > -4
    np.testing.assert_allclose(h_pos[keep], (gb / 2 * (1 + np.tanh(gb / 2)))[keep], rtol=1e-13)


def test_silu_printed_values():
    """sigma(1) = 0.7310585786300049 and sigma(2) = 0.8807970779778823 (logistic tables)."""
    g = np.zeros((1, 128)); g[0, 0] = 1.0; g[0, 1] = 2.0; g[0, 2] = -1.0
    u = np.ones((1, 128)); u[0, 1] = 3.0
    h = swiglu.swiglu_f64(gu_of(g, u))
    assert abs(h[0, 0] - 0.7310585786300049) < 1e-15
    assert abs(h[0, 1] - 3 * 2 * 0.8807970779778823) < 1e-14
    assert abs(h[0, 2] - (-1 + 0.7310585786300049)) < 1e-15
    assert h[0, 3] == 0.0


def test_extreme_arguments():
    g = np.zeros((1, 128)); g[0, 0] = -1e4; g[0, 1] = 1e4; g[0, 2] = -100.0
    u = np.full((1, 128), 2.0)
    h = swiglu.swiglu_f64(gu_of(g, u))
    gb = quant.bf16_to_f32(bf16(g))
    assert h[0, 0] == 0.0 and np.signbit(h[0, 0])               # -1e4 * 2 / inf = -0
    assert h[0, 1] == 2.0 * float(gb[0, 1])                    # e^-1e4 underflows to 0
    assert abs(h[0, 2] - (-200.0 * math.exp(-100.0) / (1 + math.exp(-100.0)))) < 1e-50


def test_gate_and_up_halves():
    """u multiplies, g gates: swapping the halves changes the result."""
    rng = np.random.default_rng(2)
    g = rng.standard_normal((2, 256))
    u = rng.standard_normal((2, 256)) * 3
    a = swiglu.swiglu_f64(gu_of(g, u))
    gb, ub = quant.bf16_to_f32(bf16(g)).astype(np.float64), quant.bf16_to_f32(bf16(u)).astype(np.float64)
    np.testing.assert_allclose(a, gb * ub / (1 + np.exp(-gb)), rtol=1e-15)
    b = swiglu.swiglu_f64(gu_of(u, g))
    assert not np.allclose(a, b)


def test_composition_with_the_pinned_quantizer():
    """On FP32 inputs that are exactly BF16 values the FP32 quantizer equals the pinned
    BF16 quantizer bit for bit; the fused oracle is that quantizer applied to RN32(h)."""
    rng = np.random.default_rng(3)
    x = bf16(rng.standard_normal((64, 384)) * 10)
    q1, s1 = quant.quantize_act_1x128(x)
    q2, s2 = swiglu.quantize_act_1x128_f32(quant.bf16_to_f32(x))
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    gu = gu_of(rng.standard_normal((8, 256)), rng.standard_normal((8, 256)))
    q, sa, h32 = swiglu.swiglu_quantize_act_1x128(gu)
    assert np.array_equal(h32, swiglu.swiglu_f64(gu).astype(np.float32))
    q3, s3 = swiglu.quantize_act_1x128_f32(h32)
    assert np.array_equal(q, q3) and np.array_equal(sa, s3)


# ------------------------------------------- the FP32-input quantizer on its own domain
#
# quantize_act_1x128_f32 serves the fused SwiGLU quantizer, whose values are FP32 products
# with 24 significant bits.  These pins compare it with the exact-rational brute force of
# test_oracle_quant (RN32(amax/448), RN32(x/s), torch's E4M3 cast) on such values, and
# check that the plausible mistakes -- rounding the values to BF16 first, or multiplying
# by RN(1/s) instead of dividing -- are caught.

from tests.test_oracle_quant import brute_quantize_group  # noqa: E402


def _brute_tiles(h32):
    M, K = h32.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((K // 128, M), np.float32)
    for m in range(M):
        for kb in range(K // 128):
            codes, sc = brute_quantize_group(h32[m, kb * 128:(kb + 1) * 128])
            q[m, kb * 128:(kb + 1) * 128] = codes
            s[kb, m] = sc
    return q, s


def _full_precision_tiles(rng, M, K):
    """FP32 values with random 24-bit significands over several binades."""
    mant = rng.integers(1 << 23, 1 << 24, size=(M, K)).astype(np.float64)
    expo = rng.integers(-30, 8, size=(M, K))
    sign = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0)
    return (sign * np.ldexp(mant, expo - 23)).astype(np.float32)


def _reciprocal_variant(h32):
    """The planted mistake: y = RN(x * RN(1/s)) instead of RN(x / s)."""
    from oracle import e4m3
    M, K = h32.shape
    t = h32.reshape(M, K // 128, 128)
    s = (np.max(np.abs(t), axis=2) / np.float32(448.0)).astype(np.float32)
    r = (np.float32(1.0) / np.where(s == 0, np.float32(1.0), s)).astype(np.float32)
    y = (t * r[:, :, None]).astype(np.float32)
    return e4m3.encode(y).reshape(M, K), s.T.copy()


def test_f32_quantizer_matches_brute_force_on_full_precision_values():
    rng = np.random.default_rng(11)
    h = _full_precision_tiles(rng, 12, 384)
    assert np.count_nonzero(quant.bf16_to_f32(wl.bf16_bits(h)) != h) > 0.99 * h.size  # not BF16 values
    q, sa = swiglu.quantize_act_1x128_f32(h)
    qb, sb = _brute_tiles(h)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    assert np.array_equal(q, qb)
    # planted mistake: rounding the FP32 values to BF16 before quantizing changes codes
    q_bf, _ = swiglu.quantize_act_1x128_f32(quant.bf16_to_f32(wl.bf16_bits(h)))
    assert np.count_nonzero(q_bf != qb) > 0


def test_f32_quantizer_special_tiles():
    rng = np.random.default_rng(12)
    h = _full_precision_tiles(rng, 6, 128)
    h[0] = 0.0                                                  # all-zero tile: s = 0, +0 codes
    h[1] = -0.0                                                 # all -0: s = 0, codes 0x80
    h[1, 5] = 0.0
    h[2] = (rng.standard_normal(128) * 1e-39).astype(np.float32)  # FP32 subnormals (no FTZ)
    h[3] = np.clip(_full_precision_tiles(rng, 1, 128)[0], -50.0, 50.0)
    h[3, 17] = np.float32(448.0 * 2.0 ** -3)                    # amax 56 = 448 * 2^-3: s = 2^-3 exactly
    h[4] = np.float32(3.0) * np.ones(128, np.float32)           # constant tile: all 0x7E
    h[5, :64] = -np.abs(h[5, :64])
    assert np.any(h[2] != 0) and np.all(np.abs(h[2]) < np.finfo(np.float32).tiny)
    q, sa = swiglu.quantize_act_1x128_f32(h)
    qb, sb = _brute_tiles(h)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    assert np.array_equal(q, qb)
    assert sa[0, 0] == 0 and np.all(q[0] == 0x00)
    assert sa[0, 1] == 0 and q[1, 5] == 0x00 and np.all(np.delete(q[1], 5) == 0x80)
    assert sa[0, 2] > 0 and sa[0, 2] < np.finfo(np.float32).tiny      # subnormal scale kept
    assert sa[0, 3] == np.float32(2.0 ** -3) and q[3, 17] == 0x7E
    assert np.all(q[4] == 0x7E)


def _division_sensitive_tile():
    """A tile (amax a, one value x) whose code differs between RN(x/s) and RN(x*RN(1/s)):
    x sits next to an E4M3 rounding boundary times s, found by search over s."""
    from oracle import e4m3
    rng = np.random.default_rng(13)
    for _ in range(200000):
        a = np.float32(rng.uniform(100.0, 400.0))
        s = np.float32(a / np.float32(448.0))
        r = np.float32(np.float32(1.0) / s)
        mid = np.float32(rng.integers(17, 31) * 0.0625 * 2.0 ** int(rng.integers(-3, 4)))  # between E4M3 codes
        base = np.float32(mid * s)
        for k in range(-3, 4):
            x = np.nextafter(base, np.float32(np.inf) if k > 0 else np.float32(-np.inf)) if k else base
            for _ in range(abs(k) - 1):
                x = np.nextafter(x, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
            x = np.float32(x)
            yd = np.float32(x / s)
            ym = np.float32(x * r)
            if e4m3.encode(np.array([yd]))[0] != e4m3.encode(np.array([ym]))[0]:
                t = np.zeros(128, np.float32)
                t[0], t[1] = a, x
                return t
    raise AssertionError("no division-sensitive tile found")


def test_f32_quantizer_divides_rather_than_multiplying_by_the_reciprocal():
    t = _division_sensitive_tile()[None, :]
    q, sa = swiglu.quantize_act_1x128_f32(t)
    qb, sb = _brute_tiles(t)
    assert np.array_equal(q, qb) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    qr, _ = _reciprocal_variant(t)
    assert qr[0, 1] != qb[0, 1]                                   # the planted mistake fails

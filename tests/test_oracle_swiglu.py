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

"""Pins for the oracle's tensor-level and delayed scalings (CPU only): equality with a
single pinned quantization group, the saturation closed form, constant tensors, and the
broadcast scale layouts the block-scaled GEMM takes (a tensor-scaled GEMM equals the
product of the tensor-dequantized operands)."""
import numpy as np

import workloads as wl
from oracle import comparators as oc
from oracle import e4m3, gemm, quant


def test_per_tensor_is_one_group():
    rng = np.random.default_rng(1)
    x = quant.bf16_to_f32(wl.bf16_bits(rng.standard_normal((64, 256)).astype(np.float32)))
    q, s = oc.per_tensor_quantize(x)
    assert s == np.float32(np.float32(np.abs(x).max()) / np.float32(448))
    q2, s2 = quant.quantize_group(x.reshape(-1))
    assert s == s2 and np.array_equal(q.reshape(-1), q2)
    assert np.count_nonzero(np.isin(q, [0x7E, 0xFE])) >= 1          # the amax lands on +-448


def test_delayed_saturation_closed_form():
    """History amax 4 -> s = 4/448; values of magnitude > 4 saturate to +-448 and are
    counted; values below keep their nearest codes."""
    x = np.array([1.0, -2.0, 4.0, 5.0, -100.0, 0.5], np.float32)
    q, s, sat, amax = oc.delayed_quantize(x, [3.0, 4.0, 2.0])
    assert s == np.float32(np.float32(4.0) / np.float32(448.0))
    assert sat == 2 and amax == np.float32(100.0)
    assert q[3] == 0x7E and q[4] == 0xFE
    ref = e4m3.encode((x[[0, 1, 2, 5]] / s).astype(np.float32))
    assert np.array_equal(q[[0, 1, 2, 5]], ref)


def test_delayed_quotient_beyond_fp32_range_saturates():
    """A stale scale far below the values: 1e30 / 1e-10 overflows FP32 and still gives the
    saturated code and is counted; 1e-3 / 1e-10 = 1e7 saturates too; zeros keep their sign."""
    x = np.array([1e30, -1e30, 1e-3, 0.0, -0.0], np.float32)
    h = np.float32(np.float32(1e-10) * np.float32(448.0))
    q, s, sat, amax = oc.delayed_quantize(x, [h])
    assert s == np.float32(h / np.float32(448.0))
    assert sat == 3 and amax == np.float32(1e30)
    assert q.tolist() == [0x7E, 0xFE, 0x7E, 0x00, 0x80]


def test_delayed_with_current_history_equals_per_tensor():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1000).astype(np.float32)
    q1, s1 = oc.per_tensor_quantize(x)
    q2, s2, sat, _ = oc.delayed_quantize(x, [np.abs(x).max()])
    assert s1 == s2 and sat == 0 and np.array_equal(q1, q2)


def test_tensor_scaled_gemm_is_dequantized_product():
    rng = np.random.default_rng(3)
    M, N, K = 40, 256, 384
    x = quant.bf16_to_f32(wl.bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    w = quant.bf16_to_f32(wl.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
    qx, sx = oc.per_tensor_quantize(x)
    qw, sw = oc.per_tensor_quantize(w)
    sa, sb = oc.broadcast_scales(sx, sw, M, N, K)
    c = gemm.gemm_blockscaled(qx, sa, qw, sb)
    ref = (e4m3.decode(qx) * float(sx)) @ (e4m3.decode(qw) * float(sw)).T
    np.testing.assert_allclose(c, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_constant_tensor():
    q, s = oc.per_tensor_quantize(np.full((8, 128), -3.0, np.float32))
    assert np.all(q == 0xFE) and s == np.float32(np.float32(3.0) / np.float32(448.0))
    assert oc.relative_error(np.ones(4) * 2.0, np.ones(4)) == 1.0

"""GPU parity of the tensor-level / delayed scaling quantizer against the oracle: codes,
scale, amax and saturated count bit-exact (tensor-level on a dense-workload slice with
outlier channels; delayed with a history amax below the current one, so outliers
saturate; an all-zero tensor; n == 0), and the tensor-scaled GEMM within the usual bound."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import comparators as oc
from oracle import gemm as og
from oracle import quant as oq

from helpers import assert_gemm_within_tol, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def run(x_bf16, scale=None):
    sc = None if scale is None else torch.tensor([scale], dtype=torch.float32, device="cuda")
    q, stats = fq.fp8q_quantize_per_tensor(dev_bf16(x_bf16), sc)
    torch.cuda.synchronize()
    return host(q), fq.tensor_stats(stats)


def test_tensor_level_dense_slice():
    x = wl.dense()["x"][:512]
    q, (amax, sat, s) = run(x)
    rq, rs = oc.per_tensor_quantize(oq.bf16_to_f32(x))
    assert np.float32(s) == rs and np.float32(amax) == np.abs(oq.bf16_to_f32(x)).max() and sat == 0
    assert np.array_equal(q, rq)


def test_delayed_saturates_outliers():
    c = wl.dense()
    x = c["x"][:512]
    xf = oq.bf16_to_f32(x)
    history = [float(np.abs(xf).max()) / 20.0, float(np.abs(xf).max()) / 25.0]
    s_in = np.float32(np.float32(max(history)) / np.float32(448.0))
    q, (amax, sat, s) = run(x, float(s_in))
    rq, rs, rsat, ramax = oc.delayed_quantize(xf, history)
    assert np.float32(s) == rs == s_in and np.float32(amax) == ramax
    assert sat == rsat and sat > 0
    assert np.array_equal(q, rq)
    print(f"\n[delayed] {sat} of {x.size} values saturated (history max 1/20 of the current amax)")


def test_delayed_quotient_beyond_fp32_range():
    """A caller's scale of ~1e-10 against values up to 1e30: quotients from below 448 to
    past the FP32 range (overflow), signed zeros; codes and count bit-exact."""
    rng = np.random.default_rng(21)
    xf = (rng.standard_normal(4096) * 3e-8).astype(np.float32)
    xf[::97] = 1e30
    xf[5::97] = -1e30
    xf[7::97] = -0.0
    xf[9::97] = 0.0
    x = wl.bf16_bits(xf)
    xr = oq.bf16_to_f32(x)
    history = [float(np.float32(1e-10) * np.float32(448.0))]
    rq, rs, rsat, ramax = oc.delayed_quantize(xr, history)
    q, (amax, sat, s) = run(x, float(rs))
    assert np.float32(s) == rs and np.float32(amax) == ramax
    assert sat == rsat and 0 < sat < x.size
    assert np.array_equal(q, rq)


def test_zero_and_empty():
    q, (amax, sat, s) = run(np.zeros((4, 128), np.uint16))
    assert amax == 0 and s == 0 and sat == 0 and np.all(q == 0)
    q, stats = fq.fp8q_quantize_per_tensor(torch.zeros(0, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert fq.tensor_stats(stats) == (0.0, 0, 0.0)


def test_tensor_scaled_gemm():
    rng = np.random.default_rng(9)
    M, N, K = 300, 384, 512
    x = wl.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qx, (_, _, sx) = run(x)
    qw, (_, _, sw) = run(w)
    sa, sb = oc.broadcast_scales(sx, sw, M, N, K)
    got = fq.fp8q_gemm_blockscaled(dev(qx), dev(sa), dev(qw), dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = og.gemm_blockscaled(qx, sa, qw, sb)
    assert_gemm_within_tol(host(got), ref, og.row_norms_act(qx, sa), og.row_norms_w(qw, sb), "tensor-scaled GEMM")

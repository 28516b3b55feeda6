"""GPU parity of the backward-pass pieces against the oracle.

* fp8q_quantize_w_128x128_t: the forward codes / scales bit-exact and the transposed
  ones bit-exact against the oracle's transposition (every byte and scale).
* fp8q_quantize_act_dual: the 1x128 codes bit-exact against the forward oracle and the
  token-tile codes / scales bit-exact against the oracle's 128x1 quantizer.
* dgrad through the block-scaled GEMM with the transposed weight operands, and wgrad
  through fp8q_gemm_rowscaled, within 2e-3 ||a_hat_row|| ||b_hat_row|| of the oracle's
  FP64 products, on shapes spanning several tiles with ragged edges, and the wgrad of a
  DeepSeek-V3 sized layer (4096 tokens, 7168 x 7168) on sampled entries.
Inputs are the oracle's codes for the GEMMs, so those tests do not depend on the GPU
quantizers."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import backward as ob
from oracle import gemm as og
from oracle import quant as oq

from helpers import assert_gemm_within_tol, assert_quant_equal, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def bf16(a):
    return wl.bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("G,N,K", [(1, 128, 128), (1, 384, 256), (3, 256, 640)])
def test_weight_quant_transposed(G, N, K):
    rng = np.random.default_rng(G * 1000 + N + K)
    w = bf16(rng.standard_normal((G, N, K)) * np.logspace(-3, 2, N)[None, :, None])
    w[0, :128, :128] = 0                                     # an all-zero block
    wq, sb, wqt, sbt = fq.fp8q_quantize_w_128x128_t(dev_bf16(w))
    torch.cuda.synchronize()
    rq, rs = oq.quantize_w_128x128(w)
    assert_quant_equal(wq, sb, rq, rs, "forward")
    tq, ts = ob.transpose_w_blocks(rq, rs)
    assert_quant_equal(wqt, sbt, tq, ts, "transposed")


def test_weight_quant_transposed_matches_plain_quantizer():
    """The transposing quantizer's forward outputs equal fp8q_quantize_w_128x128's."""
    c = wl.tiny()
    w = dev_bf16(c["w"])
    a = fq.fp8q_quantize_w_128x128(w)
    b = fq.fp8q_quantize_w_128x128_t(w)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("M,K", [(128, 128), (256, 384), (640, 256), (384, 1152)])
def test_act_quant_dual(M, K):
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)) * np.logspace(-2, 2, K)[None, :]
    x[:128, 128 - 1] = 0.0                                   # an all-zero token tile
    x[5, :128] = 0.0                                         # an all-zero channel tile
    x[300 % M, 7] = 5e4                                      # an outlier
    x = bf16(x)
    xq, sa, xqt, sat = fq.fp8q_quantize_act_dual(dev_bf16(x))
    torch.cuda.synchronize()
    rq, rs = oq.quantize_act_1x128(x)
    assert_quant_equal(xq, sa, rq, rs, "1x128 along K")
    tq, ts = ob.quantize_act_128x1(x)
    assert_quant_equal(xqt, sat, tq, ts, "128 tokens along M")


def test_act_quant_dual_matches_plain_quantizer():
    c = wl.dense()
    x = dev_bf16(c["x"][:1024])
    a = fq.fp8q_quantize_act_1x128(x)
    b = fq.fp8q_quantize_act_dual(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    tq, ts = ob.quantize_act_128x1(c["x"][:1024])
    assert_quant_equal(b[2], b[3], tq, ts, "dense rows 0..1023, token tiles")


@pytest.mark.parametrize("M,N,K", [(40, 384, 256), (300, 640, 1152), (257, 256, 896)])
def test_dgrad(M, N, K):
    """dX [M][K] = dY [M][N] . W [N][K] through the forward GEMM with the W^T operands."""
    rng = np.random.default_rng(M * 7 + N + K)
    dyq, sa = oq.quantize_act_1x128(bf16(rng.standard_normal((M, N)) * 3.0))
    wq, sb = oq.quantize_w_128x128(bf16(rng.standard_normal((N, K)) * 0.02))
    wqt, sbt = ob.transpose_w_blocks(wq, sb)
    ref = ob.dgrad(dyq, sa, wq, sb)
    got = fq.fp8q_gemm_blockscaled(dev(dyq), dev(sa), dev(wqt), dev(sbt), out_dtype=torch.float32)
    torch.cuda.synchronize()
    xn = og.row_norms_act(dyq, sa)
    wn = np.linalg.norm(oq.dequant_w(wqt, sbt), axis=1)
    assert_gemm_within_tol(host(got), ref, xn, wn, f"dgrad {M}x{N}x{K}")


def test_dgrad_from_gpu_quantizers():
    """The whole dgrad path on the GPU (dY quantized on the GPU, W through the transposing
    quantizer), compared with the oracle run on the same BF16 inputs."""
    rng = np.random.default_rng(77)
    M, N, K = 256, 512, 384
    dy = bf16(rng.standard_normal((M, N)))
    w = bf16(rng.standard_normal((N, K)) * 0.05)
    dyq, sa = fq.fp8q_quantize_act_1x128(dev_bf16(dy))
    _, _, wqt, sbt = fq.fp8q_quantize_w_128x128_t(dev_bf16(w))
    got = fq.fp8q_gemm_blockscaled(dyq, sa, wqt, sbt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rs = oq.quantize_act_1x128(dy)
    wq, sb = oq.quantize_w_128x128(w)
    ref = ob.dgrad(rq, rs, wq, sb)
    assert_gemm_within_tol(host(got), ref, og.row_norms_act(rq, rs),
                           np.linalg.norm(oq.dequant_w(wq, sb), axis=0), "dgrad GPU path")


@pytest.mark.parametrize("P,Q,Kc", [(128, 128, 128), (300, 384, 640), (257, 640, 1024), (40, 256, 256)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_rowscaled(P, Q, Kc, out_dtype):
    rng = np.random.default_rng(P + Q * 3 + Kc)
    aq, sa = oq.quantize_act_1x128(bf16(rng.standard_normal((P, Kc)) * np.logspace(-1, 1, Kc)[None, :]))
    bq, sb = oq.quantize_act_1x128(bf16(rng.standard_normal((Q, Kc)) * 4.0))
    ref = ob.gemm_rowscaled(aq, sa, bq, sb)
    got = fq.fp8q_gemm_rowscaled(dev(aq), dev(sa), dev(bq), dev(sb), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert_gemm_within_tol(host(got).astype(np.float64), ref, ob.row_norms_rowscaled(aq, sa),
                           ob.row_norms_rowscaled(bq, sb), f"rowscaled {P}x{Q}x{Kc}")


def test_wgrad_from_gpu_quantizers():
    """The whole wgrad path on the GPU: dY and X through the dual quantizer, then
    dW = dY^T X by the row-scaled GEMM; oracle on the same BF16 inputs."""
    rng = np.random.default_rng(78)
    M, N, K = 512, 384, 256
    dy = bf16(rng.standard_normal((M, N)) * np.linspace(0.1, 3, M)[:, None])
    x = bf16(rng.standard_normal((M, K)))
    _, _, dyqt, sdy = fq.fp8q_quantize_act_dual(dev_bf16(dy))
    _, _, xqt, sx = fq.fp8q_quantize_act_dual(dev_bf16(x))
    got = fq.fp8q_gemm_rowscaled(dyqt, sdy, xqt, sx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rdy, rsdy = ob.quantize_act_128x1(dy)
    rx, rsx = ob.quantize_act_128x1(x)
    ref = ob.wgrad(rdy, rsdy, rx, rsx)
    assert_gemm_within_tol(host(got), ref, ob.row_norms_rowscaled(rdy, rsdy), ob.row_norms_rowscaled(rx, rsx),
                           "wgrad GPU path")


def test_wgrad_full_size_sampled():
    """dW of a 7168x7168 layer over 4096 tokens (the dense workload's X and a seeded
    gradient), in the benchmarked launch; 4096 sampled entries against the oracle's
    per-entry FP64 dot products, plus run-to-run bit equality."""
    c = wl.dense()
    M, K = c["x"].shape
    N = 7168
    rng = np.random.default_rng(2024)
    dy = bf16(rng.standard_normal((M, N), dtype=np.float32))
    _, _, dyqt, sdy = fq.fp8q_quantize_act_dual(dev_bf16(dy))
    _, _, xqt, sx = fq.fp8q_quantize_act_dual(dev_bf16(c["x"]))
    got = fq.fp8q_gemm_rowscaled(dyqt, sdy, xqt, sx)
    again = fq.fp8q_gemm_rowscaled(dyqt, sdy, xqt, sx)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), again.view(torch.int16))
    rdy, rsdy = ob.quantize_act_128x1(dy)
    rx, rsx = ob.quantize_act_128x1(c["x"])
    assert np.array_equal(host(dyqt), rdy) and np.array_equal(host(xqt), rx)
    rows = rng.integers(0, N, 4096)
    cols = rng.integers(0, K, 4096)
    a = oq.dequant_act(rdy[np.unique(rows)], rsdy[:, np.unique(rows)])
    ai = {int(r): i for i, r in enumerate(np.unique(rows))}
    b = oq.dequant_act(rx[np.unique(cols)], rsx[:, np.unique(cols)])
    bi = {int(q): i for i, q in enumerate(np.unique(cols))}
    ref = np.array([a[ai[int(r)]] @ b[bi[int(q)]] for r, q in zip(rows, cols)])
    tol = og.TOL_REL * np.linalg.norm(a, axis=1)[[ai[int(r)] for r in rows]] * \
        np.linalg.norm(b, axis=1)[[bi[int(q)] for q in cols]]
    g = host(got)[rows, cols]
    err = np.abs(g - ref)
    print(f"\n[wgrad 7168x7168 over 4096 tokens] max |err|/tol = {np.max(err / tol):.4f}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("P,Q,Kc", [(300, 1152, 512), (257, 640, 384)])
def test_gemm_rowscaled_tile_plans(P, Q, Kc, monkeypatch):
    """The row-scaled GEMM uses the dense tile plans too (uniform 256-wide tiles or a
    256/192-wide column split); every plan meets the bar and all are bit-identical."""
    rng = np.random.default_rng(P * 3 + Q + Kc)
    aq, sa = oq.quantize_act_1x128(bf16(rng.standard_normal((P, Kc))))
    bq, sb = oq.quantize_act_1x128(bf16(rng.standard_normal((Q, Kc)) * 2.0))
    ref = ob.gemm_rowscaled(aq, sa, bq, sb)
    outs = {}
    for plan in ["off", "0", "1", "2", "auto"]:
        monkeypatch.setenv("FP8Q_DENSE_SPLIT", plan)
        got = fq.fp8q_gemm_rowscaled(dev(aq), dev(sa), dev(bq), dev(sb), out_dtype=torch.float32)
        torch.cuda.synchronize()
        outs[plan] = host(got)
        assert_gemm_within_tol(outs[plan], ref, ob.row_norms_rowscaled(aq, sa), ob.row_norms_rowscaled(bq, sb),
                               f"rowscaled {P}x{Q}x{Kc} plan {plan}")
    for plan in outs:
        assert np.array_equal(outs[plan], outs["off"]), plan

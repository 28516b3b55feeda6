"""The FP32 promotion tripwire (tests/promotion_bound.py): a second, much tighter gate than
the 2e-3 * ||x_hat|| * ||w_hat|| acceptance bound, for FP32 output on operands whose block
sums the matrix core computes exactly, so that only the promotion's rounding remains.

CPU: an emulation of FP32 promotion in ascending K-block order meets the bound, and
emulations that are about ten times less accurate (scale product or accumulator kept with
20 significant bits instead of 24, partials rounded to BF16, a partial folded twice, a
neighbouring block's scale) break it -- so a K-loop regression of that size cannot pass.
GPU: the dense, grouped and row-scaled GEMMs meet the bound (FP32 output) on shapes with
one K block, many K blocks (up to 512), ragged M and N, a column split across both tile widths, and
the ping-pong kernel's short-tile rounds."""
import numpy as np
import pytest
import torch

import promotion_bound as pb


def f32(a):
    return np.asarray(a, np.float64).astype(np.float32)


def round_bits(a, bits):
    """Round float64 values to `bits` significant bits (nearest)."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.round(m * (1 << bits)) / (1 << bits), e)


def emulate(xq, sa, wq, sb, scale_bits=24, acc_bits=24, partial_bf16=False, fold_twice=False, wrong_block=False):
    """FP32 promotion of exact block partials, ascending kb: acc = RN(t * P + acc), t = RN(sa*sb);
    the keyword arguments plant the inaccuracies the tripwire must catch."""
    P = pb.block_partials(xq, wq)
    KB, M, N = P.shape
    sbn = np.repeat(sb, 128, axis=0)                                  # [N][KB] float32
    acc = np.zeros((M, N), np.float32)
    for kb in range(KB):
        kb_s = (kb + 1) % KB if wrong_block else kb
        t = f32(sa[kb_s][:, None].astype(np.float32) * sbn[:, kb_s][None, :])
        if scale_bits < 24:
            t = f32(round_bits(t, scale_bits))
        p = P[kb]
        if partial_bf16:
            p = round_bits(p, 8)
        acc = f32(t.astype(np.float64) * p + acc.astype(np.float64))
        if fold_twice and kb == KB // 2:
            acc = f32(t.astype(np.float64) * p + acc.astype(np.float64))
        if acc_bits < 24:
            acc = f32(round_bits(acc, acc_bits))
    return acc.astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(96, 256, 128), (64, 256, 1024), (48, 128, 7168)])
def test_tripwire_passes_fp32_promotion_and_catches_regressions(M, N, K):
    xq, sa, wq, sb, C, bound = pb.dense_case(M, N, K, seed=M + N + K)
    good = emulate(xq, sa, wq, sb)
    assert pb.check(good, C, bound, f"emulated FP32 promotion {M}x{N}x{K}") <= 1.0
    for kw in ({"scale_bits": 20}, {"acc_bits": 20}, {"partial_bf16": True}, {"fold_twice": True},
               {"wrong_block": True}):
        if K == 128 and ("acc_bits" in kw or "fold_twice" in kw or "wrong_block" in kw):
            continue  # one block: no accumulator rounding beyond the first fold, no other block
        bad = emulate(xq, sa, wq, sb, **kw)
        assert np.any(np.abs(bad - C) > bound), f"{kw} not caught at {M}x{N}x{K}"


def test_tripwire_is_far_tighter_than_the_acceptance_bound():
    """On these operands the acceptance bound 2e-3 * ||x_hat|| * ||w_hat|| is more than
    10^4 times the promotion bound: a promotion 10x less accurate than FP32 passes it."""
    from oracle import gemm as og
    xq, sa, wq, sb, C, bound = pb.dense_case(64, 256, 1024, seed=4)
    tol = og.tolerance(og.row_norms_act(xq, sa), og.row_norms_w(wq, sb))
    assert np.median(tol / bound) > 1e4
    bad = emulate(xq, sa, wq, sb, scale_bits=20)
    assert np.all(np.abs(bad - C) <= tol)                             # the coarse gate misses it


# ------------------------------------------------------------------------------ GPU

@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(96, 256, 128), (257, 640, 384), (300, 1152, 1024), (512, 512, 7168),
                                   (1, 128, 2048), (600, 2304, 896), (64, 256, 65536)])
def test_gpu_dense_meets_promotion_bound(M, N, K):
    import fp8_fine_grained_fp8q_amd as fq
    from helpers import dev, host
    xq, sa, wq, sb, C, bound = pb.dense_case(M, N, K, seed=3 * M + N + K)
    c = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pb.check(host(c), C, bound, f"dense {M}x{N}x{K}")


@pytest.mark.gpu
@pytest.mark.parametrize("kernel,width", [("pp", "256"), ("pp", "224"), ("split", "256")])
def test_gpu_dense_kernels_meet_promotion_bound(kernel, width, monkeypatch):
    import fp8_fine_grained_fp8q_amd as fq
    from helpers import dev, host
    monkeypatch.setenv("FP8Q_DENSE_KERNEL", kernel)
    monkeypatch.setenv("FP8Q_PP_WIDTH", width)
    xq, sa, wq, sb, C, bound = pb.dense_case(600, 768, 3072, seed=78)
    c = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pb.check(host(c), C, bound, f"dense kernel {kernel}")


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(3072, 4096, 512), (4096, 7168, 256), (2048, 4096, 256), (1024, 4096, 512)])
def test_gpu_dense_two_region_plan_meets_promotion_bound(M, N, K):
    """Shapes the ping-pong kernel runs with a round of 192-, 128- or 64-row tiles."""
    import fp8_fine_grained_fp8q_amd as fq
    from helpers import dev, host
    xq, sa, wq, sb, C, bound = pb.dense_case(M, N, K, seed=5 * M + N + K)
    c = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pb.check(host(c), C, bound, f"dense plan {M}x{N}x{K}")


@pytest.mark.gpu
@pytest.mark.parametrize("plan", ["off", "1", "auto"])
def test_gpu_dense_plans_meet_promotion_bound(plan, monkeypatch):
    import fp8_fine_grained_fp8q_amd as fq
    from helpers import dev, host
    monkeypatch.setenv("FP8Q_DENSE_SPLIT", plan)
    xq, sa, wq, sb, C, bound = pb.dense_case(300, 1152, 2048, seed=77)
    c = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pb.check(host(c), C, bound, f"dense plan {plan}")


@pytest.mark.gpu
def test_gpu_grouped_meets_promotion_bound():
    import fp8_fine_grained_fp8q_amd as fq
    from helpers import dev, host
    sizes = [0, 1, 127, 128, 129, 300, 0, 513]
    G, N, K = len(sizes), 384, 1024
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    M = int(offsets[-1])
    rng = np.random.default_rng(5)
    xq = pb.int_codes((M, K), rng)
    wq = pb.int_codes((G, N, K), rng)
    sa = pb.full_mantissa_scales((K // 128, M), rng)
    sb = pb.full_mantissa_scales((G, N // 128, K // 128), rng)
    c = fq.fp8q_grouped_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), dev(offsets), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = host(c)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        P = pb.block_partials(xq[lo:hi], wq[g])
        sbn = np.repeat(sb[g].astype(np.float64), 128, axis=0)
        scale = sa[:, lo:hi].astype(np.float64)[:, :, None] * sbn.T[:, None, :]
        C, bound = pb.exact_and_bound(P, scale)
        pb.check(got[lo:hi], C, bound, f"grouped expert {g} ({hi - lo} rows)")


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (384, 1152, 2048)])
def test_gpu_rowscaled_meets_promotion_bound(M, N, K):
    import fp8_fine_grained_fp8q_amd as fq
    from helpers import dev, host
    aq, sa, bq, sb, C, bound = pb.rowscaled_case(M, N, K, seed=M + 2 * N + K)
    c = fq.fp8q_gemm_rowscaled(dev(aq), dev(sa), dev(bq), dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pb.check(host(c), C, bound, f"rowscaled {M}x{N}x{K}")

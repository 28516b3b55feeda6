"""GPU parity of the block-scaled FP8 GEMMs against the oracle's FP64 dequantized product.

Bar: |C_gpu - C| <= 2e-3 * ||x_hat_m||_2 * ||w_hat_n||_2 per element, C_gpu as stored
(BF16 rounding included).  The GEMM inputs are the oracle's quantized codes and scales, so
these tests do not depend on the GPU quantizers.  Cases: the tiny workload, ragged shapes
spanning several 256x256 tiles with partial tails in M and N, an exactly representable
integer case (bit-exact, pins the MFMA operand and output layouts), a characterisation of
the matrix core's own block summation, the dense 4096x7168x7168
workload in the benchmarked launch (every output), a 65536-long contraction (512 K blocks), grouped MoE shapes with
empty / 1 / 127..257-row experts and with 65..256 experts (several offset-scan chunks), the
MoE up/down workloads (every expert on sampled column blocks; four experts in full), run-to-run
determinism, the dense tile plans (uniform 256-wide tiles or a 256/192-wide column split,
bit-identical to each other) and untouched rows outside every expert range."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import gemm as og
from oracle import quant as oq

from helpers import assert_gemm_within_tol, assert_quant_equal, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def quantized(M, N, K, seed, G=None, xscale=1.0):
    rng = np.random.default_rng(seed)
    x = wl.bf16_bits(rng.standard_normal((M, K), dtype=np.float32) * np.float32(xscale))
    shape = (N, K) if G is None else (G, N, K)
    w = wl.bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02))
    return (*oq.quantize_act_1x128(x), *oq.quantize_w_128x128(w))


def gpu_gemm(xq, sa, wq, sb, out_dtype=torch.bfloat16):
    c = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(c).astype(np.float64)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_tiny(out_dtype):
    c = wl.tiny()
    xq, sa = oq.quantize_act_1x128(c["x"])
    wq, sb = oq.quantize_w_128x128(c["w"][0])
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    got = gpu_gemm(xq, sa, wq, sb, out_dtype)
    assert_gemm_within_tol(got, ref, og.row_norms_act(xq, sa), og.row_norms_w(wq, sb), "tiny")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 384, 256), (255, 256, 640), (257, 640, 384),
                                   (300, 1152, 1024), (513, 384, 128), (64, 2304, 896), (130, 256, 65536)])
def test_ragged_shapes(M, N, K):
    xq, sa, wq, sb = quantized(M, N, K, seed=M + N + K, xscale=3.0)
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    xn, wn = og.row_norms_act(xq, sa), og.row_norms_w(wq, sb)
    assert_gemm_within_tol(gpu_gemm(xq, sa, wq, sb), ref, xn, wn, f"{M}x{N}x{K} bf16")
    assert_gemm_within_tol(gpu_gemm(xq, sa, wq, sb, torch.float32), ref, xn, wn, f"{M}x{N}x{K} f32")


def test_exact_small_integers():
    """Unit scales and small integer codes whose products all lie in [-64, 64]: every
    block partial is an integer far inside FP32's exact range and inside the matrix core's
    exact range, so the GPU result must equal the oracle exactly.  A transposed or
    mis-paired operand layout, or a wrong output mapping, shows up as a mismatch here.
    The 448 entries that pin every scale to 1 are placed where they only meet zeros."""
    M, N, K = 48, 256, 384
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    w = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    x[:, ::128] = 448.0          # activation tile amax -> scale 1
    w[:, ::128] = 0.0            # ... meets only zeros
    w[127::128, 127::128] = 448.0  # weight block amax -> scale 1
    x[:, 127::128] = 0.0         # ... meets only zeros
    xq, sa = oq.quantize_act_1x128(wl.bf16_bits(x))
    wq, sb = oq.quantize_w_128x128(wl.bf16_bits(w))
    assert np.all(sa == 1.0) and np.all(sb == 1.0)
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    got = gpu_gemm(xq, sa, wq, sb, torch.float32)
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first {bad[0][0]},{bad[1][0]}: {got[bad][0]} vs {ref[bad][0]}"


def test_block_partial_precision_with_a_dominant_product():
    """Characterises the FP8 matrix core's own summation of one block's 128 products:
    each block holds one product 448*448 = 200704 and 127 products of magnitude <= 64
    (unit scales, so the exact result is an integer well inside FP32's exact range).  The
    hardware's sum is not exact in this case (the small products lose low-order bits
    against the large one), which is the accumulation-precision limit the promotion scheme
    is about; the result must still meet the acceptance bound.  Prints the observed error."""
    M, N, K = 48, 256, 384
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    w = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    x[:, ::128] = 448.0
    w[::128, ::128] = 448.0
    xq, sa = oq.quantize_act_1x128(wl.bf16_bits(x))
    wq, sb = oq.quantize_w_128x128(wl.bf16_bits(w))
    assert np.all(sa == 1.0) and np.all(sb == 1.0)
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    got = gpu_gemm(xq, sa, wq, sb, torch.float32)
    dom = np.zeros(N, bool)
    dom[::128] = True
    err = np.abs(got - ref)
    print(f"\n[block-partial precision] rows with a 200704 product per block: max |err| "
          f"{err[:, dom].max():g} (of |C| ~ {np.abs(ref[:, dom]).max():g}); other rows max |err| {err[:, ~dom].max():g}")
    assert_gemm_within_tol(got, ref, og.row_norms_act(xq, sa), og.row_norms_w(wq, sb), "dominant product")


PLANS = ["off", "0", "1", "2", "auto"]


@pytest.mark.parametrize("M,N,K", [(300, 1152, 1024), (257, 640, 384), (40, 128, 256)])
def test_dense_tile_plans(M, N, K, monkeypatch):
    """Dense launches either use 256-wide tiles throughout ("off") or split the columns
    into a 256-wide range [0, a*256) and a 192-wide range after it (a = 0, 1, 2), one
    workgroup index range each; "auto" is the library's own choice.  Every plan must meet
    the bar, and since a tile's width does not change the arithmetic of any output (same
    block partials, same FMA order), all plans must give bit-identical results."""
    xq, sa, wq, sb = quantized(M, N, K, seed=7 * M + N + K, xscale=2.0)
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    xn, wn = og.row_norms_act(xq, sa), og.row_norms_w(wq, sb)
    outs = {}
    for plan in PLANS:
        monkeypatch.setenv("FP8Q_DENSE_SPLIT", plan)
        outs[plan] = gpu_gemm(xq, sa, wq, sb, torch.float32)
        assert_gemm_within_tol(outs[plan], ref, xn, wn, f"{M}x{N}x{K} plan {plan}")
    for plan in PLANS[1:]:
        assert np.array_equal(outs[plan], outs["off"]), plan


@pytest.mark.parametrize("width", ["256", "224"])
@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 1152, 1024), (257, 640, 384), (40, 128, 256),
                                   (513, 768, 2176), (1024, 1024, 7168), (260, 2688, 512)])
def test_dense_pingpong_kernel(M, N, K, width, monkeypatch):
    """The ping-pong kernel (256 x 256 or 256 x 224 tiles, the two waves of a SIMD
    alternating between LDS reads and MFMAs) against the oracle bound, and bit-identical to
    the column-split kernel: the same block partials folded in the same order.  224-wide
    tiles put wave columns across 128-column weight-scale blocks (N = 2688 = 12 x 224)."""
    xq, sa, wq, sb = quantized(M, N, K, seed=11 * M + N + K, xscale=2.0)
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    xn, wn = og.row_norms_act(xq, sa), og.row_norms_w(wq, sb)
    monkeypatch.setenv("FP8Q_PP_WIDTH", width)
    monkeypatch.setenv("FP8Q_DENSE_KERNEL", "pp")
    pp32 = gpu_gemm(xq, sa, wq, sb, torch.float32)
    ppbf = gpu_gemm(xq, sa, wq, sb)
    monkeypatch.setenv("FP8Q_DENSE_KERNEL", "split")
    sp32 = gpu_gemm(xq, sa, wq, sb, torch.float32)
    spbf = gpu_gemm(xq, sa, wq, sb)
    assert_gemm_within_tol(pp32, ref, xn, wn, f"pp {M}x{N}x{K} f32")
    assert_gemm_within_tol(ppbf, ref, xn, wn, f"pp {M}x{N}x{K} bf16")
    assert np.array_equal(pp32, sp32)
    assert np.array_equal(ppbf, spbf)


@pytest.mark.parametrize("M,N,K", [(4096, 7168, 128), (4096, 7168, 1024), (3072, 4096, 512), (8192, 7168, 128),
                                   (2048, 4096, 256), (1024, 4096, 512), (4096, 4096, 256)])
def test_dense_two_region_plan(M, N, K, monkeypatch):
    """The ping-pong kernel's two-region plan: with 256 CUs a last round of 256 x 256 tiles
    that is 3/4, 1/2 or 1/4 full runs as one round of 192-, 128- or 64-row tiles.  4096x7168
    (448 tiles): rows 3072.. of columns 0..4095 and all rows of 4096.. in 256-row tiles,
    then rows 0..3071 of columns 0..4095 in 192-row tiles; 3072x4096 (192 tiles) is that
    round alone; 8192x7168 (896 tiles) ends in 128-row tiles; 2048x4096 (128) and 1024x4096
    (64) become one round of 128- and 64-row tiles; 4096x4096 (256 tiles, one whole round)
    keeps uniform tiles.  Every output against the oracle bound, bit-identical to the
    uniform tiles (FP8Q_PP_PLAN=off), both output types."""
    xq, sa, wq, sb = quantized(M, N, K, seed=13 * M + N + K, xscale=2.0)
    ref = og.gemm_blockscaled(xq, sa, wq, sb)
    xn, wn = og.row_norms_act(xq, sa), og.row_norms_w(wq, sb)
    monkeypatch.setenv("FP8Q_DENSE_KERNEL", "pp")
    plan32 = gpu_gemm(xq, sa, wq, sb, torch.float32)
    planbf = gpu_gemm(xq, sa, wq, sb)
    monkeypatch.setenv("FP8Q_PP_PLAN", "off")
    uni32 = gpu_gemm(xq, sa, wq, sb, torch.float32)
    unibf = gpu_gemm(xq, sa, wq, sb)
    assert_gemm_within_tol(plan32, ref, xn, wn, f"plan {M}x{N}x{K} f32")
    assert_gemm_within_tol(planbf, ref, xn, wn, f"plan {M}x{N}x{K} bf16")
    assert np.array_equal(plan32, uni32)
    assert np.array_equal(planbf, unibf)


def test_deterministic():
    xq, sa, wq, sb = quantized(300, 640, 512, seed=5)
    a = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb))
    b = fq.fp8q_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.fixture(scope="module")
def dense_quantized():
    c = wl.dense()
    xq, sa = oq.quantize_act_1x128(c["x"])
    wq, sb = oq.quantize_w_128x128(c["w"][0])
    return xq, sa, wq, sb


def test_dense_full_size(dense_quantized):
    """The 4096x7168x7168 workload in the benchmarked launch, every output checked against
    the oracle (an FP64 product of the dequantized operands: a few seconds on the host)."""
    xq, sa, wq, sb = dense_quantized
    got = gpu_gemm(xq, sa, wq, sb)
    xh = oq.dequant_act(xq, sa)
    wh = oq.dequant_w(wq, sb)
    ref = xh @ wh.T
    assert_gemm_within_tol(got, ref, np.linalg.norm(xh, axis=1), np.linalg.norm(wh, axis=1), "dense 4096x7168x7168")


def test_dense_full_size_repeatable(dense_quantized):
    """Ten launches at full size give bit-identical output (no cross-wave races in the
    LDS pipeline; the kernel has no atomics or split reductions)."""
    xq, sa, wq, sb = (dev(a) for a in dense_quantized)
    first = fq.fp8q_gemm_blockscaled(xq, sa, wq, sb)
    for _ in range(9):
        again = fq.fp8q_gemm_blockscaled(xq, sa, wq, sb)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_dense_full_size_plans_agree(dense_quantized, monkeypatch):
    """At full size the benchmarked (automatic) plan and the uniform 256-wide plan give
    bit-identical output."""
    xq, sa, wq, sb = (dev(a) for a in dense_quantized)
    auto = fq.fp8q_gemm_blockscaled(xq, sa, wq, sb)
    monkeypatch.setenv("FP8Q_DENSE_SPLIT", "off")
    uniform = fq.fp8q_gemm_blockscaled(xq, sa, wq, sb)
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int16), uniform.view(torch.int16))


def run_grouped(xq, sa, wq, sb, offsets, out_dtype=torch.bfloat16, fill=None):
    M, N = xq.shape[0], wq.shape[1]
    out = None
    if fill is not None:
        out = torch.full((M, N), fill, dtype=out_dtype, device="cuda")
    c = fq.fp8q_grouped_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), dev(offsets),
                                         out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    return host(c).astype(np.float64)


@pytest.mark.parametrize("sizes", [[0, 1, 127, 128, 129, 255, 256, 257], [300], [0, 0, 5, 0],
                                   [513, 2, 0, 260]])
def test_grouped_edge_sizes(sizes):
    G, N, K = len(sizes), 384, 256
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    M = int(offsets[-1])
    xq, sa, wq, sb = quantized(M, N, K, seed=sum(sizes) + G, G=G, xscale=2.0)
    ref = og.grouped_gemm_blockscaled(xq, sa, wq, sb, offsets)
    got = run_grouped(xq, sa, wq, sb, offsets)
    xn = og.row_norms_act(xq, sa)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            wn = og.row_norms_w(wq[g], sb[g])
            assert_gemm_within_tol(got[lo:hi], ref[lo:hi], xn[lo:hi], wn, f"expert {g} ({hi - lo} rows)")


def _grouped_sizes(G, seed, zero=(), fixed=None):
    rng = np.random.default_rng(seed)
    sizes = rng.integers(0, 48, size=G)
    sizes[list(zero)] = 0
    for g, n in (fixed or {}).items():
        sizes[g] = n
    return sizes


@pytest.mark.parametrize("G,zero,fixed", [
    # one expert past the first 64-expert chunk; the last expert of the first chunk empty
    (65, (63,), {64: 130, 0: 257}),
    # empty experts on both sides of the chunk boundary, ragged tails <= 128 and > 128 rows
    (128, (62, 63, 64, 65), {66: 100, 127: 257, 1: 129}),
    # four chunks, empty experts around every boundary, the very last expert non-empty
    (256, (63, 64, 127, 128, 191, 192), {193: 1, 255: 129, 100: 300, 200: 128}),
    # all experts of the first chunk empty: every row lives in later chunks
    (130, tuple(range(64)), {64: 200, 129: 5}),
])
def test_grouped_many_experts(G, zero, fixed):
    """More experts than one scan chunk (the kernel scans the offsets 64 experts at a
    time): experts found in later chunks, empty experts at chunk edges, ragged tails."""
    sizes = _grouped_sizes(G, seed=G, zero=zero, fixed=fixed)
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    M, N, K = int(offsets[-1]), 256, 256
    xq, sa, wq, sb = quantized(M, N, K, seed=G + 1, G=G, xscale=2.0)
    ref = og.grouped_gemm_blockscaled(xq, sa, wq, sb, offsets)
    got = run_grouped(xq, sa, wq, sb, offsets, out_dtype=torch.float32, fill=-777.0)
    xn = og.row_norms_act(xq, sa)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            assert_gemm_within_tol(got[lo:hi], ref[lo:hi], xn[lo:hi], og.row_norms_w(wq[g], sb[g]),
                                   f"G={G} expert {g} ({hi - lo} rows)")
    assert not np.any(got == -777.0)


def test_grouped_single_expert_equals_dense():
    xq, sa, wq, sb = quantized(300, 640, 384, seed=21)
    dense = gpu_gemm(xq, sa, wq, sb)
    grouped = run_grouped(xq, sa, wq[None], sb[None], np.array([0, 300], np.int32))
    assert np.array_equal(dense, grouped)


def test_grouped_rows_outside_ranges_untouched():
    """offsets[G] < M_tot: the trailing rows belong to no expert and keep their contents."""
    G, N, K = 2, 256, 256
    xq, sa, wq, sb = quantized(200, N, K, seed=8, G=G)
    offsets = np.array([0, 70, 150], np.int32)
    got = run_grouped(xq, sa, wq, sb, offsets, out_dtype=torch.float32, fill=-777.0)
    assert np.all(got[150:] == -777.0)
    ref = og.grouped_gemm_blockscaled(xq, sa, wq, sb, offsets)
    xn = og.row_norms_act(xq, sa)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        assert_gemm_within_tol(got[lo:hi], ref[lo:hi], xn[lo:hi], og.row_norms_w(wq[g], sb[g]), f"expert {g}")


def test_grouped_debug_offsets_check(monkeypatch):
    """With FP8Q_DEBUG set, valid offsets give the same result as without the check and
    invalid ones (first != 0, decreasing, last != M_tot) return FP8Q_ERR_OFFSETS with
    nothing written; FP8Q_DEBUG=0 turns the check off again."""
    G, N, K, M = 3, 256, 256, 200
    xq, sa, wq, sb = quantized(M, N, K, seed=31, G=G)
    good = np.array([0, 60, 130, 200], np.int32)
    plain = run_grouped(xq, sa, wq, sb, good)
    monkeypatch.setenv("FP8Q_DEBUG", "1")
    assert np.array_equal(run_grouped(xq, sa, wq, sb, good), plain)
    for bad in ([1, 60, 130, 200], [0, 130, 60, 200], [0, 60, 130, 199]):
        out = torch.full((M, N), -5.0, dtype=torch.float32, device="cuda")
        with pytest.raises(fq.Fp8qError) as err:
            fq.fp8q_grouped_gemm_blockscaled(dev(xq), dev(sa), dev(wq), dev(sb), dev(np.array(bad, np.int32)),
                                             out_dtype=torch.float32, out=out)
        assert err.value.status == fq.FP8Q_ERR_OFFSETS, bad
        torch.cuda.synchronize()
        assert bool(torch.all(out == -5.0)), bad
    monkeypatch.setenv("FP8Q_DEBUG", "0")
    run_grouped(xq, sa, wq, sb, np.array([0, 130, 60, 200], np.int32))  # clamped, no check


@pytest.mark.parametrize("name", ["moe_up", "moe_down"])
def test_moe_workloads_all_experts(name):
    """Full-size MoE workloads, every one of the 32 experts checked: all of its rows
    against two 128-column blocks of its output (a different pair per expert, so the
    experts together cover every column block and both tile shapes' positions).  The GPU
    quantizes everything; the rows of X and the sampled weight blocks are also quantized by
    the oracle, must equal the GPU's codes bit for bit, and are what the reference uses."""
    c = wl.CONFIGS[name]()
    offsets = c["offsets"]
    x_d = dev_bf16(c["x"])
    w_d = dev_bf16(c["w"])
    xq_d, sa_d = fq.fp8q_quantize_act_1x128(x_d)
    wq_d, sb_d = fq.fp8q_quantize_w_128x128(w_d)
    out = fq.fp8q_grouped_gemm_blockscaled(xq_d, sa_d, wq_d, sb_d, dev(offsets))
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    xq, sa = oq.quantize_act_1x128(c["x"])
    assert_quant_equal(xq_d, sa_d, xq, sa, f"{name} activations")
    G, N, K = c["w"].shape
    NB = N // 128
    xh = oq.dequant_act(xq, sa)
    checked = 0
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        for nb in sorted({g % NB, (7 * g + NB // 2 + 3) % NB}):
            wq_b, sb_b = oq.quantize_w_128x128(c["w"][g, nb * 128:(nb + 1) * 128])
            assert_quant_equal(wq_d[g, nb * 128:(nb + 1) * 128], sb_d[g, nb:nb + 1], wq_b, sb_b,
                               f"{name} expert {g} weight block row {nb}")
            if hi == lo:
                continue
            wh = oq.dequant_w(wq_b, sb_b)
            assert_gemm_within_tol(got[lo:hi, nb * 128:(nb + 1) * 128], xh[lo:hi] @ wh.T,
                                   np.linalg.norm(xh[lo:hi], axis=1), np.linalg.norm(wh, axis=1),
                                   f"{name} expert {g} cols {nb * 128}..{nb * 128 + 127}")
            checked += hi - lo
    assert checked >= int(offsets[-1])


@pytest.mark.parametrize("name", ["moe_up", "moe_down"])
def test_moe_workloads_sampled(name):
    """Full-size MoE workloads (32 local experts, routed token counts).  Four experts (first,
    two middle, last non-empty) are checked row by row against the oracle.  Their GEMM
    inputs are the oracle's codes and scales; the other experts' inputs come from the GPU
    quantizers (their outputs are not checked), and for the sampled experts the GPU
    quantizers' output must equal the oracle's bit for bit."""
    c = wl.CONFIGS[name]()
    offsets = c["offsets"]
    x_d = dev_bf16(c["x"])
    w_d = dev_bf16(c["w"])
    xq_d, sa_d = fq.fp8q_quantize_act_1x128(x_d)
    wq_d, sb_d = fq.fp8q_quantize_w_128x128(w_d)
    torch.cuda.synchronize()
    nz = [g for g in range(len(offsets) - 1) if offsets[g + 1] > offsets[g]]
    pick = sorted(set([nz[0], nz[len(nz) // 3], nz[2 * len(nz) // 3], nz[-1]]))
    ref_in = {}
    for g in pick:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        xq_g, sa_g = oq.quantize_act_1x128(c["x"][lo:hi])
        wq_g, sb_g = oq.quantize_w_128x128(c["w"][g])
        assert_quant_equal(xq_d[lo:hi], sa_d[:, lo:hi].contiguous(), xq_g, sa_g, f"{name} act rows of expert {g}")
        assert_quant_equal(wq_d[g], sb_d[g], wq_g, sb_g, f"{name} weights of expert {g}")
        xq_d[lo:hi] = dev(xq_g)
        sa_d[:, lo:hi] = dev(sa_g)
        wq_d[g] = dev(wq_g)
        sb_d[g] = dev(sb_g)
        ref_in[g] = (xq_g, sa_g, wq_g, sb_g)
    off_d = dev(offsets)
    out = fq.fp8q_grouped_gemm_blockscaled(xq_d, sa_d, wq_d, sb_d, off_d)
    for _ in range(3):  # repeatable at full size
        again = fq.fp8q_grouped_gemm_blockscaled(xq_d, sa_d, wq_d, sb_d, off_d)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    got = host(out).astype(np.float64)
    for g in pick:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        xq_g, sa_g, wq_g, sb_g = ref_in[g]
        xh = oq.dequant_act(xq_g, sa_g)
        wh = oq.dequant_w(wq_g, sb_g)
        assert_gemm_within_tol(got[lo:hi], xh @ wh.T, np.linalg.norm(xh, axis=1),
                               np.linalg.norm(wh, axis=1), f"{name} expert {g}")


def test_binding_rejects_inconsistent_shapes():
    """The binding checks every buffer's shape against the sizes it passes to the C ABI
    (plain pointers there), so a mismatched scale or output tensor never reaches a kernel."""
    xq, sa, wq, sb = (dev(a) for a in quantized(64, 256, 256, seed=1))
    with pytest.raises(ValueError):
        fq.fp8q_gemm_blockscaled(xq, sa[:1], wq, sb)
    with pytest.raises(ValueError):
        fq.fp8q_gemm_blockscaled(xq, sa, wq, sb[:1])
    with pytest.raises(ValueError):
        fq.fp8q_gemm_blockscaled(xq, sa, wq, sb, out=torch.empty((64, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fq.fp8q_quantize_act_1x128(torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda"),
                                   sa=torch.empty((1, 64), device="cuda"))
    with pytest.raises(ValueError):
        fq.fp8q_grouped_gemm_blockscaled(xq, sa, wq[None], sb[None], torch.zeros(3, dtype=torch.int32, device="cuda"))

"""GPU parity of the online quantizers: codes and scales bit-exact with the oracle.

Inputs are the seeded workloads (tiny and dense at full size) plus constructed tiles that
cover every BF16 value against a spread of scales (both division paths of the kernel),
zero / signed-zero / subnormal / power-of-two / constant groups and ragged row counts; the
fused entry point (both quantizers in one launch) against the oracle and against the two
separate launches."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import quant as oq

from helpers import assert_quant_equal, dev_bf16

pytestmark = pytest.mark.gpu


def run_act(x_u16):
    xq, sa = fq.fp8q_quantize_act_1x128(dev_bf16(x_u16))
    torch.cuda.synchronize()
    return xq, sa


def run_w(w_u16):
    wq, sb = fq.fp8q_quantize_w_128x128(dev_bf16(w_u16))
    torch.cuda.synchronize()
    return wq, sb


def test_act_tiny():
    x = wl.tiny()["x"]
    xq, sa = run_act(x)
    assert_quant_equal(xq, sa, *oq.quantize_act_1x128(x), what="tiny act")


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (15, 384), (16, 128), (17, 512), (33, 1024), (100, 640)])
def test_act_ragged_rows(M, K):
    rng = np.random.default_rng(M * 1000 + K)
    x = wl.bf16_bits(rng.standard_normal((M, K), dtype=np.float32) * np.float32(rng.uniform(0.01, 100)))
    xq, sa = run_act(x)
    assert_quant_equal(xq, sa, *oq.quantize_act_1x128(x), what=f"act {M}x{K}")


def test_act_special_tiles():
    rows = []
    z = np.zeros(128, np.float32)
    rows.append(z.copy())                                    # all +0
    t = z.copy(); t[[3, 70, 127]] = -0.0; rows.append(t)     # signed zeros only
    t = z.copy(); t[5] = -0.0; t[9] = 3.0; rows.append(t)    # -0 next to a value
    rows.append(np.full(128, 7.5, np.float32))               # constant
    rows.append(np.full(128, -1e-30, np.float32))            # constant, tiny
    t = np.linspace(-1, 1, 128).astype(np.float32) * 448 * 2.0 ** -20; rows.append(t)  # power-of-two amax
    t = np.linspace(-1, 1, 128).astype(np.float32) * 448 * 2.0 ** 40; rows.append(t)
    rows.append((np.arange(128) - 64).astype(np.float32) * np.float32(2.0 ** -133))  # BF16 subnormals
    rows.append(np.full(128, 3.0e38, np.float32))            # near the top of the range
    t = z.copy(); t[0] = 2.84375; t[1] = 8.058547973632812e-05; rows.append(t)  # division vs reciprocal case
    x = wl.bf16_bits(np.stack(rows))
    x = np.concatenate([x, x[::-1]], axis=1)                 # K = 256, reversed copy in tile 2
    xq, sa = run_act(x)
    assert_quant_equal(xq, sa, *oq.quantize_act_1x128(x), what="special tiles")


def _all_bf16_tiles(amax_bits):
    """Tiles whose first element is amax and whose other 127 elements run through every
    finite BF16 value of magnitude <= amax (both signs)."""
    tiles = []
    for ab in amax_bits:
        vals = np.arange(0, ab + 1, dtype=np.uint32).astype(np.uint16)
        vals = np.concatenate([vals, vals | np.uint16(0x8000)])
        n = (len(vals) + 126) // 127
        pad = np.zeros(n * 127, np.uint16)
        pad[:len(vals)] = vals
        body = pad.reshape(n, 127)
        tiles.append(np.concatenate([np.full((n, 1), ab, np.uint16), body], axis=1))
    return np.concatenate(tiles, axis=0)


def test_act_every_bf16_value_against_many_scales():
    rng = np.random.default_rng(7)
    exps = [1, 2, 30, 60, 62, 63, 64, 65, 66, 80, 100, 120, 126, 127, 128, 129, 130, 134, 140,
            160, 180, 190, 191, 192, 193, 200, 230, 253, 254]
    amax_bits = []
    for e in exps:
        for m in (0, 1, 0x3F, 0x40, 0x7F, int(rng.integers(0, 128))):
            amax_bits.append((e << 7) | m)
    amax_bits += [1, 2, 0x7F, 0x80]                          # subnormal and smallest normal amax
    x = _all_bf16_tiles(sorted(set(amax_bits)))
    # several tiles per row: reshape to rows of 4 tiles (pad with zero tiles)
    rows = (x.shape[0] + 3) // 4
    pad = np.zeros((rows * 4, 128), np.uint16)
    pad[:x.shape[0]] = x
    x = pad.reshape(rows, 512)
    assert x.size > 4_000_000
    xq, sa = run_act(x)
    assert_quant_equal(xq, sa, *oq.quantize_act_1x128(x), what="every bf16 value x scale grid")


def test_act_dense_full_size():
    c = wl.dense()
    x = c["x"]
    xq, sa = run_act(x)
    assert_quant_equal(xq, sa, *oq.quantize_act_1x128(x), what="dense act 4096x7168")


def test_act_deterministic_and_no_overrun():
    x = wl.tiny()["x"][:37]
    d = dev_bf16(x)
    xq = torch.full((37 + 8, 512), 0xA5, dtype=torch.uint8, device="cuda")
    sa = torch.full((4 * 37 + 16,), 1234.5, dtype=torch.float32, device="cuda")
    fq.fp8q_quantize_act_1x128(d, xq=xq[:37], sa=sa[:4 * 37].view(4, 37))
    first = xq.clone()
    fq.fp8q_quantize_act_1x128(d, xq=xq[:37], sa=sa[:4 * 37].view(4, 37))
    torch.cuda.synchronize()
    assert torch.equal(first, xq)
    assert torch.all(xq[37:] == 0xA5) and torch.all(sa[4 * 37:] == 1234.5)


def test_w_tiny():
    w = wl.tiny()["w"]
    wq, sb = run_w(w)
    assert_quant_equal(wq, sb, *oq.quantize_w_128x128(w), what="tiny weights")


def test_w_grouped_and_special_blocks():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((3, 384, 256), dtype=np.float32) * np.float32(0.02)
    w[0, :128, :128] = 0.0                                   # zero block
    w[0, :128, 128:] = -0.0                                  # signed-zero block
    w[1, 128:256, :128] *= np.float32(2.0 ** -130)           # subnormal block
    w[2, 256:, 128:] = 5.0                                   # constant block
    w[1, 0:128, 128:256] *= np.float32(1e25)                 # large block (slow division path)
    wb = wl.bf16_bits(w)
    wq, sb = run_w(wb)
    assert_quant_equal(wq, sb, *oq.quantize_w_128x128(wb), what="grouped special weights")


def test_w_dense_full_size():
    w = wl.dense()["w"]
    wq, sb = run_w(w)
    assert_quant_equal(wq, sb, *oq.quantize_w_128x128(w), what="dense weights 7168x7168")


@pytest.mark.parametrize("M,G,N,K", [(17, 1, 256, 384), (300, 3, 128, 640), (0, 2, 256, 256), (33, 1, 0, 512)])
def test_fused_act_w_matches_oracle(M, G, N, K):
    """Both quantizers in one launch: the same codes and scales as the oracle (ragged rows,
    several experts, and each half empty in turn)."""
    rng = np.random.default_rng(M * 7 + G * 5 + N + K)
    x = wl.bf16_bits(rng.standard_normal((M, K), dtype=np.float32) * np.float32(3.0))
    w = wl.bf16_bits(rng.standard_normal((G, N, K), dtype=np.float32) * np.float32(0.02))
    xq, sa, wq, sb = fq.fp8q_quantize_act_w(dev_bf16(x), dev_bf16(w))
    torch.cuda.synchronize()
    if M:
        assert_quant_equal(xq, sa, *oq.quantize_act_1x128(x), what=f"fused act {M}x{K}")
    if N:
        assert_quant_equal(wq, sb, *oq.quantize_w_128x128(w), what=f"fused weights {G}x{N}x{K}")


def test_fused_act_w_equals_separate_calls_full_size():
    """At the dense workload's full size the fused launch writes exactly what the two
    separate quantizer launches write."""
    c = wl.dense()
    x, w = dev_bf16(c["x"]), dev_bf16(c["w"][0])
    xq1, sa1 = fq.fp8q_quantize_act_1x128(x)
    wq1, sb1 = fq.fp8q_quantize_w_128x128(w)
    xq2, sa2, wq2, sb2 = fq.fp8q_quantize_act_w(x, w)
    torch.cuda.synchronize()
    assert torch.equal(xq1, xq2) and torch.equal(wq1, wq2)
    assert torch.equal(sa1.view(torch.int32), sa2.view(torch.int32))
    assert torch.equal(sb1.view(torch.int32), sb2.view(torch.int32))

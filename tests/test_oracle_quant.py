"""Pins for the oracle's online 1x128 / 128x128 quantizers (CPU only).

Fixed by: a pure-Python brute force that divides exactly in rationals and
rounds once to FP64 and once to FP32 (double rounding is innocuous for a
quotient when the wider format has at least 2p+2 bits: Figueroa, "When is
double rounding innocuous?", 1995) with torch's E4M3 cast for the codes; the
invariants the method implies (the amax element lands on +-448, scaling by
2^j, row / block locality, transpose symmetry, dequantization within half an
E4M3 step); closed forms (power-of-two amax, constant tiles); the hand-worked
tile in tests/golden/act_tile_example.txt."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import e4m3, quant

GOLDEN_TILE = os.path.join(os.path.dirname(__file__), "golden", "act_tile_example.txt")


def torch_encode(y):
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def f32_exact_quotient(a: float, b: float) -> np.float32:
    """RN32(a/b) via an exact rational quotient (double rounding through FP64 is innocuous)."""
    return np.float32(float(Fraction(a) / Fraction(b)))


def brute_quantize_group(vals):
    """One tile / block by the definition, element by element in pure Python."""
    vals = [float(v) for v in vals]
    amax = max(abs(v) for v in vals)
    s = f32_exact_quotient(amax, 448.0)
    if s == 0:
        ys = np.array(vals, dtype=np.float32)
    else:
        ys = np.array([f32_exact_quotient(v, float(s)) for v in vals], dtype=np.float32)
    return torch_encode(ys), s


def bits_to_f32(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- brute force

def test_act_quant_matches_brute_force_tiny():
    c = wl.tiny()
    x = c["x"][:32]                                   # 32 rows x 4 tiles
    q, sa = quant.quantize_act_1x128(x)
    xf = bits_to_f32(x)
    for m in range(x.shape[0]):
        for kb in range(x.shape[1] // 128):
            codes, s = brute_quantize_group(xf[m, kb * 128:(kb + 1) * 128])
            assert sa[kb, m].view(np.uint32) == np.float32(s).view(np.uint32), (m, kb)
            assert np.array_equal(q[m, kb * 128:(kb + 1) * 128], codes), (m, kb)


def test_weight_quant_matches_brute_force_tiny():
    c = wl.tiny()
    w = c["w"][0]                                     # 256 x 512 -> 2 x 4 blocks
    q, sb = quant.quantize_w_128x128(w)
    wf = bits_to_f32(w)
    for nb in range(2):
        for kb in range(4):
            blk = wf[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            codes, s = brute_quantize_group(blk.reshape(-1))
            assert sb[nb, kb].view(np.uint32) == np.float32(s).view(np.uint32)
            assert np.array_equal(q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].reshape(-1), codes)


def test_group_function_equals_vectorised_form():
    rng = np.random.default_rng(3)
    x = wl.bf16_bits(rng.standard_normal((7, 384), dtype=np.float32) * 3)
    q, sa = quant.quantize_act_1x128(x)
    xf = bits_to_f32(x)
    for m in range(7):
        for kb in range(3):
            cq, cs = quant.quantize_group(xf[m, kb * 128:(kb + 1) * 128])
            assert cs == sa[kb, m]
            assert np.array_equal(cq, q[m, kb * 128:(kb + 1) * 128])


# ---------------------------------------------------------------- fixtures and closed forms

def _golden_tile():
    x = np.zeros(128, dtype=np.float32)
    want = np.zeros(128, dtype=np.uint8)
    scale = None
    with open(GOLDEN_TILE) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# scale"):
                scale = float.fromhex(line.split()[2])
            if not line or line.startswith("#"):
                continue
            pos, v, c = line.split()[:3]
            x[int(pos)] = float.fromhex(v)
            want[int(pos)] = int(c, 16)
    return x, want, scale


def test_golden_hand_worked_tile():
    x, want, scale = _golden_tile()
    xb = wl.bf16_bits(x)
    assert np.array_equal(bits_to_f32(xb).view(np.uint32), x.view(np.uint32))  # exact in BF16
    q, sa = quant.quantize_act_1x128(xb[None, :])
    assert sa[0, 0] == np.float32(scale)
    assert np.array_equal(q[0], want), [(i, hex(q[0, i]), hex(want[i])) for i in np.nonzero(q[0] != want)[0]]


@pytest.mark.parametrize("j", [-135, -60, -10, 0, 3, 20, 100])
def test_power_of_two_amax_gives_exact_scale(j):
    """amax = 448 * 2^j -> s = 2^j exactly, and each code is E4M3(x * 2^-j)."""
    rng = np.random.default_rng(j + 1000)
    amax = np.float32(448.0) * np.float32(2.0) ** j if j > -130 else np.float32(448.0 * 2.0 ** j)
    if not np.isfinite(amax) or amax == 0:
        pytest.skip("outside FP32")
    x = (rng.uniform(-1, 1, 128) * float(amax)).astype(np.float32)
    x[17] = amax
    xb = wl.bf16_bits(x)
    xf = bits_to_f32(xb)
    q, sa = quant.quantize_act_1x128(xb[None])
    assert sa[0, 0] == np.float32(2.0 ** j)
    want = torch_encode(np.array([f32_exact_quotient(float(v), 2.0 ** j) for v in xf], np.float32))
    assert np.array_equal(q[0], want)
    assert q[0, 17] == 0x7E


def test_constant_tile():
    for c in [1.0, -3.25, 1e-20, 7e30]:
        xb = wl.bf16_bits(np.full((2, 256), c, np.float32))
        cb = float(bits_to_f32(xb)[0, 0])
        q, sa = quant.quantize_act_1x128(xb)
        assert np.all(q == (0xFE if c < 0 else 0x7E))
        assert np.all(sa == f32_exact_quotient(abs(cb), 448.0))


def test_zero_and_signed_zero_tile():
    x = np.zeros((1, 256), np.float32)
    x[0, 3] = -0.0
    x[0, 200] = -0.0
    x[0, 130] = 2.0
    xb = wl.bf16_bits(x)
    q, sa = quant.quantize_act_1x128(xb)
    assert sa[0, 0] == 0 and sa[1, 0] == np.float32(2.0 / 448.0)
    assert q[0, 3] == 0x80 and q[0, 200] == 0x80 and q[0, 0] == 0x00 and q[0, 130] == 0x7E
    assert np.count_nonzero(q[0, :128] == 0x80) == 1


def test_subnormal_tile():
    """A tile whose amax is a BF16 subnormal: the scale is an FP32 subnormal (no flush)."""
    u = np.arange(1, 129, dtype=np.uint16)            # BF16 subnormal patterns 1..128
    xf = bits_to_f32(u)
    q, sa = quant.quantize_act_1x128(u[None])
    assert 0 < sa[0, 0] < np.float32(2.0 ** -126)
    codes, s = brute_quantize_group(xf)
    assert sa[0, 0] == s
    assert np.array_equal(q[0], codes)
    assert q[0, 127] == 0x7E


def test_division_not_reciprocal_multiply():
    """The reading y = RN(x / s): a case where multiplying by RN(1/s) changes the code."""
    amax, x = 2.84375, 8.058547973632812e-05
    tile = np.zeros(128, np.float32)
    tile[0], tile[1] = amax, x
    xb = wl.bf16_bits(tile)
    assert bits_to_f32(xb)[1] == np.float32(x)
    q, sa = quant.quantize_act_1x128(xb[None])
    s = sa[0, 0]
    by_div = torch_encode(np.array([f32_exact_quotient(x, float(s))], np.float32))[0]
    by_rcp = torch_encode(np.array([np.float32(x) * (np.float32(1) / s)], np.float32))[0]
    assert by_div != by_rcp
    assert q[0, 1] == by_div == 0x06


def test_fp32_division_is_correctly_rounded_here():
    """The oracle's numpy FP32 division (incl. subnormal quotients and divisors) equals the
    exact quotient rounded once; guards against flush-to-zero or approximate division."""
    u = np.arange(1, 0x7F80, 3, dtype=np.uint32).astype(np.uint16)
    xs = bits_to_f32(u)
    for s in [np.float32(2.0 ** -140), np.float32(1.0 / 448), np.float32(3.0), np.float32(7.77e-3),
              np.float32(1.234e20)]:
        with np.errstate(over="ignore"):
            got = xs / s
            ref = (xs.astype(np.float64) / np.float64(s)).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- invariants

def test_amax_element_maps_to_448():
    c = wl.tiny()
    x = c["x"]
    q, sa = quant.quantize_act_1x128(x)
    xf = bits_to_f32(x).reshape(128, 4, 128)
    am = np.argmax(np.abs(xf), axis=2)
    qq = q.reshape(128, 4, 128)
    top = np.take_along_axis(qq, am[:, :, None], 2)[:, :, 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    assert np.array_equal(sa.T, np.max(np.abs(xf), axis=2) / np.float32(448))
    w = c["w"]
    wq, sb = quant.quantize_w_128x128(w)
    wf = bits_to_f32(w[0]).reshape(2, 128, 4, 128).transpose(0, 2, 1, 3).reshape(2, 4, -1)
    wqq = wq[0].reshape(2, 128, 4, 128).transpose(0, 2, 1, 3).reshape(2, 4, -1)
    am = np.argmax(np.abs(wf), axis=2)
    top = np.take_along_axis(wqq, am[:, :, None], 2)[:, :, 0]
    assert np.all((top == 0x7E) | (top == 0xFE))


def test_dequantized_within_half_e4m3_step():
    c = wl.tiny()
    q, sa = quant.quantize_act_1x128(c["x"])
    xf = bits_to_f32(c["x"]).astype(np.float64)
    y = (bits_to_f32(c["x"]).reshape(128, 4, 128) / sa.T[:, :, None]).reshape(128, 512)
    err = np.abs(e4m3.decode(q) - y.astype(np.float64))
    assert np.all(err <= e4m3.half_ulp(y))
    xh = quant.dequant_act(q, sa)
    s_full = np.repeat(sa.T, 128, axis=1).astype(np.float64)
    assert np.all(np.abs(xh - xf) <= e4m3.half_ulp(y) * s_full * (1 + 2.0 ** -20) + 1e-300)


@pytest.mark.parametrize("j", [-30, -3, 1, 17])
def test_power_of_two_scaling_invariance(j):
    c = wl.tiny()
    x = bits_to_f32(c["x"])
    x2 = (x * np.float32(2.0 ** j)).astype(np.float32)
    x2b = wl.bf16_bits(x2)
    assert np.array_equal(bits_to_f32(x2b), x2)               # exact, no rounding
    q1, s1 = quant.quantize_act_1x128(c["x"])
    q2, s2 = quant.quantize_act_1x128(x2b)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(2.0 ** j))


def test_row_permutation_and_block_locality():
    c = wl.tiny()
    x = c["x"]
    perm = np.random.default_rng(9).permutation(x.shape[0])
    q1, s1 = quant.quantize_act_1x128(x)
    q2, s2 = quant.quantize_act_1x128(x[perm])
    assert np.array_equal(q2, q1[perm]) and np.array_equal(s2, s1[:, perm])
    w = c["w"][0]
    wq, sb = quant.quantize_w_128x128(w)
    sub_q, sub_s = quant.quantize_w_128x128(w[128:256, 256:512])
    assert np.array_equal(sub_q, wq[128:256, 256:512]) and np.array_equal(sub_s, sb[1:2, 2:4])
    tq, ts = quant.quantize_w_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(tq, wq.T) and np.array_equal(ts, sb.T)


def test_act_tiles_are_along_k():
    """A tile is one row's 128 consecutive channels: an outlier changes only its own tile."""
    x = np.ones((3, 384), np.float32)
    x[1, 200] = 1000.0
    q, sa = quant.quantize_act_1x128(wl.bf16_bits(x))
    assert sa[1, 1] == np.float32(1000.0 / 448.0)
    mask = np.ones_like(sa, bool)
    mask[1, 1] = False
    assert np.all(sa[mask] == np.float32(1.0 / 448.0))


def test_rejects_bad_shapes_and_non_finite():
    with pytest.raises(ValueError):
        quant.quantize_act_1x128(np.zeros((2, 100), np.uint16))
    with pytest.raises(ValueError):
        quant.quantize_w_128x128(np.zeros((100, 128), np.uint16))
    bad = np.zeros((1, 128), np.uint16)
    bad[0, 5] = 0x7F80                                 # +inf
    with pytest.raises(ValueError):
        quant.quantize_act_1x128(bad)

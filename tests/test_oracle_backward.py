"""Pins for the oracle's backward-pass pieces (CPU only): transposed weight blocks, the
128x1 token-tile quantizer and the GEMM with per-row scales on both operands.

Fixed by: the direct products of the dequantized originals (dX = dY_hat W_hat with no
transposition anywhere, dW = dY_hat^T X_hat from the token-tile dequantization done in
the original layout), a pure-Python rational brute force of the 128x1 tiles and of a
tiny wgrad, a closed form for constant operands, and shape / orientation checks that a
transposed or swapped operand would fail."""
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from oracle import backward as ob
from oracle import e4m3, quant

from test_oracle_quant import bits_to_f32, brute_quantize_group


def bf16(a):
    return wl.bf16_bits(np.asarray(a, dtype=np.float32))


def dequant_tokens_direct(x_bf16):
    """128x1 tiles dequantized in the original [M][C] layout, tile by tile with the
    brute-force quantizer (pure Python per tile)."""
    xf = bits_to_f32(x_bf16)
    M, C = xf.shape
    out = np.zeros((M, C))
    for c in range(C):
        for mb in range(M // 128):
            codes, s = brute_quantize_group(xf[mb * 128:(mb + 1) * 128, c])
            out[mb * 128:(mb + 1) * 128, c] = e4m3.decode(codes) * float(s)
    return out


def test_token_tiles_match_brute_force():
    rng = np.random.default_rng(11)
    x = bf16(rng.standard_normal((256, 5)) * np.array([1e-3, 1.0, 30.0, 0.02, 5e3]))
    q, s = ob.quantize_act_128x1(x)
    assert q.shape == (5, 256) and s.shape == (2, 5)
    xf = bits_to_f32(x)
    for c in range(5):
        for mb in range(2):
            codes, sc = brute_quantize_group(xf[mb * 128:(mb + 1) * 128, c])
            assert s[mb, c].view(np.uint32) == np.float32(sc).view(np.uint32), (mb, c)
            assert np.array_equal(q[c, mb * 128:(mb + 1) * 128], codes), (mb, c)


def test_token_tiles_reject_ragged_token_count():
    with pytest.raises(ValueError):
        ob.quantize_act_128x1(np.zeros((200, 128), np.uint16))


def test_token_tile_scale_is_column_amax():
    """A column whose largest magnitude sits in token 77 of the second tile: that tile's
    scale is |x|/448 and the element encodes to +-448 (0x7e / 0xfe)."""
    x = np.zeros((256, 128), np.float32)
    x[128 + 77, 3] = -896.0
    x[128 + 5, 3] = 2.0
    x[10, 3] = 1.0
    q, s = ob.quantize_act_128x1(bf16(x))
    assert s[1, 3] == np.float32(2.0) and s[0, 3] == np.float32(1.0 / 448.0)
    assert q[3, 128 + 77] == 0xFE and q[3, 10] == 0x7E
    assert s[0, 4] == 0 and np.all(q[4] == 0)


def test_dgrad_equals_direct_product():
    """dgrad through the transposed blocks equals dY_hat @ W_hat with W_hat dequantized in
    its own [N][K] layout (a swapped or untransposed block or scale fails this)."""
    rng = np.random.default_rng(5)
    M, N, K = 40, 384, 256
    dyq, sa = quant.quantize_act_1x128(bf16(rng.standard_normal((M, N))))
    w = rng.standard_normal((N, K)) * np.linspace(0.01, 3.0, N)[:, None] * np.linspace(1, 7, K)[None, :]
    wq, sb = quant.quantize_w_128x128(bf16(w))
    wqt, sbt = ob.transpose_w_blocks(wq, sb)
    assert wqt.shape == (K, N) and sbt.shape == (K // 128, N // 128)
    got = ob.dgrad(dyq, sa, wq, sb)
    ref = quant.dequant_act(dyq, sa) @ quant.dequant_w(wq, sb)
    assert got.shape == (M, K)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_wgrad_equals_direct_product():
    """wgrad from the channel-major token-tile codes equals dY_hat^T X_hat with both
    dequantized tile by tile in the original token-major layout."""
    rng = np.random.default_rng(6)
    M, N, K = 256, 128, 256
    dy = bf16(rng.standard_normal((M, N)) * np.linspace(0.1, 4.0, M)[:, None])
    x = bf16(rng.standard_normal((M, K)))
    dyq_t, s_dy = ob.quantize_act_128x1(dy)
    xq_t, s_x = ob.quantize_act_128x1(x)
    got = ob.wgrad(dyq_t, s_dy, xq_t, s_x)
    assert got.shape == (N, K)
    ref = dequant_tokens_direct(dy).T @ dequant_tokens_direct(x)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_wgrad_rational_brute_force_tiny():
    """Every entry of a 3x2 wgrad over 128 tokens as an exact rational sum."""
    rng = np.random.default_rng(9)
    dy = bf16(rng.standard_normal((128, 3)))
    x = bf16(rng.standard_normal((128, 2)) * 10)
    dyq_t, s_dy = ob.quantize_act_128x1(dy)
    xq_t, s_x = ob.quantize_act_128x1(x)
    got = ob.wgrad(dyq_t, s_dy, xq_t, s_x)
    for n in range(3):
        for k in range(2):
            acc = Fraction(0)
            for m in range(128):
                acc += (Fraction(float(e4m3.decode(dyq_t[n, m]))) * Fraction(float(s_dy[0, n]))
                        * Fraction(float(e4m3.decode(xq_t[k, m]))) * Fraction(float(s_x[0, k])))
            assert abs(got[n, k] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc))), (n, k)


def test_wgrad_constant_closed_form():
    """dY = a, X = b everywhere: every element is its tile's amax, so it encodes to +-448
    and dequantizes to +-448 s with s = RN32(|v|/448); dW = M (448 s_dY)(-448 s_X), which
    is a b up to the two scale roundings."""
    M, N, K = 384, 128, 256
    dyq_t, s_dy = ob.quantize_act_128x1(bf16(np.full((M, N), 0.5)))
    xq_t, s_x = ob.quantize_act_128x1(bf16(np.full((M, K), -4.0)))
    assert np.all(dyq_t == 0x7E) and np.all(xq_t == 0xFE)
    got = ob.wgrad(dyq_t, s_dy, xq_t, s_x)
    want = M * (448.0 * float(s_dy[0, 0])) * (-448.0 * float(s_x[0, 0]))
    np.testing.assert_allclose(got, want, rtol=1e-14)
    np.testing.assert_allclose(want, M * 0.5 * -4.0, rtol=1e-7)

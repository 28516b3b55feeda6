"""Online fine-grained quantizers: 1x128 activation tiles and 128x128 weight blocks.

Follows: dtcms.com DeepSeek-V3 page, section 3.2 (fine-grained quantization:
1x128 tiles / 128x128 blocks, each scaled on its own); codingmall.com page on
FP8 in DeepSeek-V3 training, sections "Dinh luong hat min" (activations in
1x128 tiles, weights in 128x128 blocks, scaled independently) and "Dinh luong
truc tuyen" (scale of every tile / block computed on the fly, no delayed
scaling from past maxima); risenshineclean.com training-algorithm page,
section 3, bullets "fine-grained quantization" (a tile is one token's 128
channels) and "online quantization".

Readings (the pages give no formula):
* scale s = RN32(amax / 448), amax = largest |x| in the tile or block, 448 the
  largest E4M3 magnitude; the scale is not rounded to a power of two;
* quantized value y = RN32(x / s) (an IEEE correctly rounded FP32 division,
  not a multiplication by a rounded reciprocal), then code = E4M3(y);
  dequantized value = decode(code) * s;
* an all-zero tile / block gets s = 0 and sign-preserving zero codes;
* FP32 subnormals are kept (no flush to zero) for s and y;
* inputs are finite BF16; a tile runs along K (the contraction dimension) of a
  row-major X[M][K]; a block is 128 consecutive rows (N) by 128 consecutive
  columns (K) of a row-major W[N][K]; K and N are multiples of 128, M is any.

Scale layouts: activation scales sa[K/128][M] (tile column major, so one
K-block's scales for consecutive rows are contiguous); weight scales
sb[G][N/128][K/128].

Parity status: pinned (closed forms, invariants, a pure-Python brute force
with exact rational division, hand-derived fixtures).
"""
from __future__ import annotations

import numpy as np

from . import e4m3

TILE = 128
BLOCK = 128
F32_448 = np.float32(448.0)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> FP32 values (a BF16 number is the top half of an FP32 one)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def quantize_group(x: np.ndarray):
    """Quantize one group of FP32 values (any shape) with one shared online scale.

    Returns (codes uint8 of x's shape, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantizer input must be finite")
    amax = np.float32(np.max(np.abs(x)))
    s = np.float32(amax / F32_448)
    if s == 0:
        return e4m3.encode(x), s  # all entries are +-0 -> 0x00 / 0x80
    y = (x / s).astype(np.float32)
    return e4m3.encode(y), s


def quantize_act_1x128(x_bf16: np.ndarray):
    """Activation quantizer.  x_bf16: uint16 [M][K] -> (xq uint8 [M][K], sa float32 [K/128][M]).

    Vectorised over tiles; per tile it is exactly ``quantize_group``."""
    x = bf16_to_f32(x_bf16)
    M, K = x.shape
    if K % TILE:
        raise ValueError("K must be a multiple of 128")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantizer input must be finite")
    t = x.reshape(M, K // TILE, TILE)
    amax = np.max(np.abs(t), axis=2)                      # [M][K/128], exact
    s = (amax / F32_448).astype(np.float32)               # RN32 division
    safe = np.where(s == 0, np.float32(1.0), s)
    y = (t / safe[:, :, None]).astype(np.float32)         # RN32 division; zero tiles: y = x = +-0
    q = e4m3.encode(y).reshape(M, K)
    sa = np.ascontiguousarray(s.T)                         # [K/128][M]
    return q, sa


def quantize_w_128x128(w_bf16: np.ndarray):
    """Weight quantizer.  w_bf16: uint16 [G][N][K] (or [N][K]) ->
    (wq uint8 same shape, sb float32 [G][N/128][K/128] (or [N/128][K/128]))."""
    squeeze = w_bf16.ndim == 2
    w = bf16_to_f32(w_bf16 if not squeeze else w_bf16[None])
    G, N, K = w.shape
    if N % BLOCK or K % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    if not np.all(np.isfinite(w)):
        raise ValueError("quantizer input must be finite")
    b = w.reshape(G, N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = np.max(np.abs(b), axis=(2, 4))                 # [G][N/128][K/128]
    s = (amax / F32_448).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s)
    y = (b / safe[:, :, None, :, None]).astype(np.float32)
    q = e4m3.encode(y).reshape(G, N, K)
    if squeeze:
        return q[0], s[0]
    return q, s


def dequant_act(xq: np.ndarray, sa: np.ndarray) -> np.ndarray:
    """x_hat[m][k] = decode(xq[m][k]) * sa[k/128][m], in float64 (exact)."""
    M, K = xq.shape
    d = e4m3.decode(xq).reshape(M, K // TILE, TILE)
    return (d * sa.T.astype(np.float64)[:, :, None]).reshape(M, K)


def dequant_w(wq: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """w_hat[g][n][k] = decode(wq[g][n][k]) * sb[g][n/128][k/128], in float64 (exact)."""
    squeeze = wq.ndim == 2
    if squeeze:
        wq, sb = wq[None], sb[None]
    G, N, K = wq.shape
    d = e4m3.decode(wq).reshape(G, N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    out = (d * sb.astype(np.float64)[:, :, None, :, None]).reshape(G, N, K)
    return out[0] if squeeze else out

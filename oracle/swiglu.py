"""SwiGLU followed by online 1x128 activation quantization (the input of the MoE expert
down-projection), fused into one pass on the GPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: the expert FFN of DeepSeek's MoE layers (risenshineclean.com training-algorithm
page, section 2: each token is processed by a few routed experts) whose down-projection
input is quantized online in 1x128 tiles like every GEMM activation (codingmall.com page,
sections "Dinh luong hat min" and "Dinh luong truc tuyen").  The pages do not name the
expert activation function; SwiGLU, h = SiLU(g) * u with SiLU(g) = g / (1 + e^-g), is the
reading used here (the up-projection output holds g and u side by side).

Readings:
* input gu[M][2I] BF16 row-major: g = gu[:, :I], u = gu[:, I:]; I a multiple of 128;
* h is formed in FP32 (no BF16 round trip between the activation and the quantizer); the
  oracle computes h in FP64 and rounds it once to FP32, then applies the 1x128 quantizer
  of quant.py to those FP32 values;
* the GPU's FP32 SiLU is not correctly rounded, so a GPU code may legitimately differ from
  the oracle's where h/s lies within a few FP32 ulps of an E4M3 rounding boundary, and a
  tile scale by a few ulps; the parity tests compare on those terms.

Parity status: pinned -- SiLU by its identities, printed logistic values and extreme
arguments; the FP32-input 1x128 quantizer by the exact-rational brute force on full-precision
FP32 tiles (24-bit significands) and on zero, -0, FP32-subnormal, power-of-two and constant
tiles, with a tile on which dividing and multiplying by RN(1/s) give different codes and
random tiles on which rounding the values to BF16 first changes codes.
"""
from __future__ import annotations

import numpy as np

from . import quant


def swiglu_f64(gu_bf16: np.ndarray) -> np.ndarray:
    """h = SiLU(g) * u in float64 for gu uint16 [M][2I] -> [M][I]."""
    x = quant.bf16_to_f32(gu_bf16).astype(np.float64)
    I = x.shape[1] // 2
    g, u = x[:, :I], x[:, I:]
    with np.errstate(over="ignore"):
        return g * u / (1.0 + np.exp(-g))


def quantize_act_1x128_f32(h32: np.ndarray):
    """The 1x128 quantizer on FP32 values [M][K] (same arithmetic as quant.quantize_act_1x128)."""
    h32 = np.asarray(h32, dtype=np.float32)
    M, K = h32.shape
    if K % quant.TILE:
        raise ValueError("K must be a multiple of 128")
    q = np.empty((M, K), np.uint8)
    sa = np.empty((K // quant.TILE, M), np.float32)
    t = h32.reshape(M, K // quant.TILE, quant.TILE)
    amax = np.max(np.abs(t), axis=2)
    s = (amax / quant.F32_448).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s)
    y = (t / safe[:, :, None]).astype(np.float32)
    from . import e4m3
    q[:] = e4m3.encode(y).reshape(M, K)
    sa[:] = s.T
    return q, sa


def swiglu_quantize_act_1x128(gu_bf16: np.ndarray):
    """-> (codes uint8 [M][I], scales float32 [I/128][M], h rounded to FP32 [M][I])."""
    h32 = swiglu_f64(gu_bf16).astype(np.float32)
    q, sa = quantize_act_1x128_f32(h32)
    return q, sa, h32

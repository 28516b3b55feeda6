"""The prior-art FP8 scalings the pages contrast online fine-grained quantization with,
for an accuracy comparison (TEST INFRASTRUCTURE ONLY, see the package docstring).

* Tensor-level scaling: one scale for a whole tensor (risenshineclean.com page, section 3,
  first bullet, which sets the 1x128 / 128x128 groups against traditional tensor-level
  quantization; codingmall.com page, section "Dinh luong hat min": per-group scales keep
  outliers from distorting the whole tensor).
* Delayed scaling: the scale comes from the largest amax seen over past steps rather than
  from the current values (codingmall.com, section "Dinh luong truc tuyen", and the
  risenshineclean.com page, section 3, bullet "online quantization", which say the online
  scheme removes the need for this).

Readings (the pages give no formula for either):
* tensor-level: s = RN32(amax(tensor) / 448), codes E4M3(RN32(x / s)) exactly as one group
  of quant.quantize_group (nearest even, saturating);
* delayed: s = RN32(max(history) / 448) with history the amax of the previous L steps
  (the current amax is not used for the current step, it is appended to the history);
  values whose quotient exceeds 448 saturate to +-448, including a quotient beyond the FP32
  range (a stale scale far below the current values), and the number of saturated elements
  is reported;
* both feed the same block-scaled GEMM with every tile / block scale equal to the tensor's
  scale, so the comparison isolates the scaling granularity.

Parity status: pinned (equality with one-group quantization, saturation closed form,
constant tensors).
"""
from __future__ import annotations

import numpy as np

from . import e4m3, quant


def per_tensor_quantize(x32: np.ndarray):
    """One scale for all of x (FP32 values, any shape) -> (codes uint8, scale float32)."""
    return quant.quantize_group(np.asarray(x32, dtype=np.float32))


def delayed_quantize(x32: np.ndarray, history):
    """Scale from the history's largest amax -> (codes, scale, saturated count, current amax)."""
    x = np.asarray(x32, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantizer input must be finite")
    h = np.float32(max(float(v) for v in history))
    s = np.float32(h / quant.F32_448)
    amax = np.float32(np.max(np.abs(x)))
    if s == 0:
        return e4m3.encode(x), s, 0, amax
    with np.errstate(over="ignore"):
        y = (x / s).astype(np.float32)
    saturated = int(np.count_nonzero(np.abs(y) > np.float32(448.0)))
    # an FP32 overflow (+-inf) saturates like any other quotient above 448
    y = np.where(np.isinf(y), np.copysign(np.float32(2 * 448.0), y), y).astype(np.float32)
    return e4m3.encode(y), s, saturated, amax


def broadcast_scales(s_x, s_w, M, N, K):
    """Tile / block scale arrays of the block-scaled GEMM, every entry the tensor's scale:
    (sa float32 [K/128][M], sb float32 [N/128][K/128])."""
    return (np.full((K // 128, M), np.float32(s_x), np.float32),
            np.full((N // 128, K // 128), np.float32(s_w), np.float32))


def relative_error(c_hat: np.ndarray, c_ref: np.ndarray) -> float:
    """||c_hat - c_ref||_F / ||c_ref||_F."""
    c_hat = np.asarray(c_hat, np.float64)
    c_ref = np.asarray(c_ref, np.float64)
    return float(np.linalg.norm(c_hat - c_ref) / np.linalg.norm(c_ref))

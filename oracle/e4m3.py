"""E4M3 (OCP "E4M3FN") decode and encode, written from the format definition.

The pages fix the format only by name: codingmall.com page on FP8 in
DeepSeek-V3 training, section "Dinh dang E4M3 hop nhat" (unified E4M3), and
risenshineclean.com DeepSeek training-algorithm page, section 3, bullet
"unified E4M3 format".  Readings taken here (the pages give no bit layout,
rounding or overflow rule):

* layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
  field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2^8 = 448 (the OCP FP8
  "E4M3FN" variant, whose maximum 448 is the divisor of the scale);
* encoding rounds to the nearest representable value, ties to the code with an
  even mantissa (its last bit 0);
* magnitudes beyond 448 saturate to 448 (never reached by the quantizers for
  finite input, whose scaled values stay below 448 * (1 + 2^-22));
* the sign is kept, so -0 and negatives that round to zero encode as 0x80.

Parity status: pinned (exhaustive decode against closed forms and torch's
float8_e4m3fn, encoder against torch's cast on dense samples of every binade
and on every midpoint, hand-derived fixtures under tests/golden/).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode_code(c: int) -> float:
    """Value of one E4M3 code, straight from the bit fields."""
    c = int(c) & 0xFF
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes in code order 0x00..0x7E; code order is value order.
_MAGS = DECODE[:0x7F].copy()
assert np.all(np.diff(_MAGS) > 0)
# Midpoints between neighbouring magnitudes (exact in float64: both ends have <= 4
# significant bits and nearby exponents).
_MIDS = (_MAGS[:-1] + _MAGS[1:]) / 2.0


def decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of uint8 codes to float64."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(y: np.ndarray) -> np.ndarray:
    """Encode FP32 values to E4M3 codes: nearest representable, ties to even, saturating.

    ``y`` must be finite.  Works element by element on any shape."""
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("E4M3 encode: input must be finite")
    a = np.abs(y).astype(np.float64)
    # lo = largest magnitude index with _MAGS[lo] <= a (clipped into the finite range)
    lo = np.searchsorted(_MAGS, a, side="right") - 1
    lo = np.clip(lo, 0, len(_MAGS) - 1)
    hi = np.minimum(lo + 1, len(_MAGS) - 1)
    mid = np.where(lo < len(_MAGS) - 1, _MIDS[np.minimum(lo, len(_MIDS) - 1)], np.inf)
    pick_hi = (a > mid) | ((a == mid) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    # saturation: anything at or above the top magnitude is the top code (0x7E)
    idx = np.where(a >= E4M3_MAX, 0x7E, idx)
    neg = np.signbit(y)
    return (idx.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def half_ulp(y: np.ndarray) -> np.ndarray:
    """Half the E4M3 spacing at |y| (the largest rounding error of a nearest encoding
    for |y| <= 448): 2^-10 in the subnormal range, 2^(e-4) in binade [2^e, 2^(e+1))."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 4)

"""Pins for the oracle's E4M3 codec (CPU only).

What fixes it: the OCP E4M3FN format definition (closed forms below), the
hand-derived fixture tests/golden/e4m3_cases.txt, and torch's own
float8_e4m3fn cast (round to nearest even, non-saturating, so it is compared
only below 464 where saturation cannot arise)."""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_cases.txt")


def torch_encode(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_closed_forms():
    assert e4m3.DECODE[0x7E] == 448.0
    assert e4m3.DECODE[0xFE] == -448.0
    assert e4m3.DECODE[0x38] == 1.0
    assert e4m3.DECODE[0x08] == 2.0 ** -6
    assert e4m3.DECODE[0x07] == 7 * 2.0 ** -9
    assert e4m3.DECODE[0x01] == 2.0 ** -9
    assert e4m3.DECODE[0x00] == 0.0 and not np.signbit(e4m3.DECODE[0x00])
    assert e4m3.DECODE[0x80] == 0.0 and np.signbit(e4m3.DECODE[0x80])
    assert np.isnan(e4m3.DECODE[0x7F]) and np.isnan(e4m3.DECODE[0xFF])
    assert np.sum(np.isnan(e4m3.DECODE)) == 2
    # every normal code: (1 + m/8) * 2^(e-7)
    for c in range(0x08, 0x7F):
        e, m = c >> 3, c & 7
        assert e4m3.DECODE[c] == (8 + m) * 2.0 ** (e - 10)
        assert e4m3.DECODE[c | 0x80] == -e4m3.DECODE[c]


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_decode(codes)
    ours = e4m3.decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def _golden_cases():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, c = line.split()[:2]
            rows.append((float.fromhex(v), int(c, 16)))
    return rows


def test_golden_hand_derived_cases():
    cases = _golden_cases()
    assert len(cases) >= 20
    vals = np.array([v for v, _ in cases], dtype=np.float32)
    want = np.array([c for _, c in cases], dtype=np.uint8)
    assert np.all(vals.astype(np.float64) == np.array([v for v, _ in cases]))  # exact in FP32
    got = e4m3.encode(vals)
    bad = [(cases[i][0], hex(want[i]), hex(got[i])) for i in np.nonzero(got != want)[0]]
    assert not bad, bad


def _dense_fp32_sample():
    """FP32 values covering every E4M3 binade and the subnormal range densely, every
    E4M3 midpoint and its 6 FP32 neighbours on each side, and random bit patterns."""
    parts = []
    for e in range(-24, 9):
        mant = np.arange(0, 1 << 23, 97, dtype=np.uint32)
        bits = ((np.uint32(e + 127) << np.uint32(23)) | mant).astype(np.uint32)
        parts.append(bits.view(np.float32))
    mags = e4m3.DECODE[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    for k in range(-6, 7):
        parts.append(np.nextafter(mids, np.float32(np.inf if k > 0 else 0)) if k else mids)
        if abs(k) > 1:
            step = mids.copy()
            for _ in range(abs(k)):
                step = np.nextafter(step, np.float32(np.inf if k > 0 else 0))
            parts.append(step)
    rng = np.random.default_rng(11)
    rb = rng.integers(0, 0x43E80000, size=2_000_000, dtype=np.uint32)  # |y| < 464
    parts.append(rb.view(np.float32))
    parts.append(np.array([0.0, 2.0 ** -149, 2.0 ** -126, 2.0 ** -10], dtype=np.float32))
    v = np.concatenate(parts)
    v = v[np.abs(v) < 464.0]
    return np.concatenate([v, -v])


def test_encoder_matches_torch_cast_below_464():
    y = _dense_fp32_sample()
    assert y.size > 5_000_000
    ours = e4m3.encode(y)
    ref = torch_encode(y)
    diff = np.nonzero(ours != ref)[0]
    assert diff.size == 0, [(float(y[i]), hex(ours[i]), hex(ref[i])) for i in diff[:10]]


def test_encoder_saturates_and_keeps_sign():
    y = np.array([448.0, 448.0001, 463.99, 464.0, 470.0, 1e30, 3.4e38], dtype=np.float32)
    assert np.all(e4m3.encode(y) == 0x7E)
    assert np.all(e4m3.encode(-y) == 0xFE)
    assert e4m3.encode(np.array([-0.0], np.float32))[0] == 0x80
    assert e4m3.encode(np.array([-1e-30], np.float32))[0] == 0x80


def test_encoder_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.inf], np.float32))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], np.float32))


def test_encode_is_nearest():
    """Brute force: the chosen code minimises |decode(code) - y| over all finite codes."""
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(20000) * rng.choice([1e-3, 1e-1, 1, 30, 200], 20000)).astype(np.float32)
    y = y[np.abs(y) <= 448]
    q = e4m3.encode(y)
    allv = e4m3.DECODE[[c for c in range(256) if c not in e4m3.NAN_CODES]]
    best = np.min(np.abs(allv[None, :] - y.astype(np.float64)[:, None]), axis=1)
    got = np.abs(e4m3.decode(q) - y.astype(np.float64))
    assert np.array_equal(best, got)


def test_half_ulp():
    assert e4m3.half_ulp(np.array([1.0]))[0] == 2.0 ** -4
    assert e4m3.half_ulp(np.array([300.0]))[0] == 16.0
    assert e4m3.half_ulp(np.array([1e-3]))[0] == 2.0 ** -10
    assert e4m3.half_ulp(np.array([2.0 ** -6]))[0] == 2.0 ** -10

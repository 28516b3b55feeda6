"""Seeded input generators: determinism, BF16 rounding and routing structure (CPU only)."""
import hashlib

import numpy as np
import torch

import workloads as wl


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_tiny_is_deterministic_and_shaped():
    a, b = wl.tiny(), wl.tiny()
    assert a["x"].shape == (128, 512) and a["w"].shape == (1, 256, 512)
    assert a["x"].dtype == np.uint16
    assert _h(a["x"]) == _h(b["x"]) and _h(a["w"]) == _h(b["w"])
    assert _h(wl.tiny(seed=99)["x"]) != _h(a["x"])
    # ~1% of entries are x50 outliers
    xf = (a["x"].astype(np.uint32) << 16).view(np.float32)
    frac = np.mean(np.abs(xf) > 8)
    assert 0.003 < frac < 0.02


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.bf16_bits(v), ref)


def test_routing_structure():
    rows, offsets = wl.routing()
    assert len(rows) == 32 and offsets.shape == (33,) and offsets[0] == 0
    assert np.all(np.diff(offsets) >= 0)
    counts = np.diff(offsets)
    # 8 of 256 experts per token -> 8192*8/256 = 256 tokens per expert on average
    assert 50 <= counts.min() and counts.max() <= 1200          # strongly uneven by design
    assert abs(counts.mean() - 256) < 40
    for r in rows:
        assert np.all(np.diff(r) > 0)          # stable, token order
    rows2, off2 = wl.routing()
    assert np.array_equal(offsets, off2)


def test_dense_outlier_channels_small():
    c = wl.dense(M=64, N=256, K=1024)
    xf = (c["x"].astype(np.uint32) << 16).view(np.float32)
    colmax = np.abs(xf).max(axis=0)
    big = np.nonzero(colmax > 50)[0]
    assert set(big.tolist()) <= set(c["outlier_channels"].tolist())
    assert len(c["outlier_channels"]) == 8

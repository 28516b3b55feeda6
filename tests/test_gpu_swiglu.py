"""GPU parity of the fused SwiGLU + 1x128 quantizer against the oracle (FP64 SwiGLU rounded
once to FP32, then the pinned quantizer).

The GPU forms SiLU in FP32 with a few ulps of error, so the comparison is: every tile scale
within 2^-20 relative of the oracle's, and every code equal to the oracle's except where the
oracle's quotient h/s lies within 2^-16 (relative) of an E4M3 rounding boundary, where the
other neighbour is also accepted; such exemptions must stay rare (< 1e-3 of the codes).
Cases: random g, u at several magnitudes with ragged row counts, extreme gate values
(+-100, 0, zero u rows, an all-zero tile), and the MoE down-projection input at full size
(8360 routed rows, I = 2048).  Gates below about -87 give h below the FP32 normal range,
which the kernel does not reproduce to this accuracy (stated in the header); the extreme
cases stay above it.""" 
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import e4m3, swiglu

from helpers import dev_bf16, host

pytestmark = pytest.mark.gpu

_POS = np.sort(np.unique(np.abs(e4m3.decode(np.arange(256, dtype=np.uint8)))))
_POS = _POS[np.isfinite(_POS)]
_MID = (_POS[1:] + _POS[:-1]) / 2  # E4M3 rounding boundaries between positive neighbours


def check(gu, what):
    M, I2 = gu.shape
    I = I2 // 2
    xq, sa = fq.fp8q_swiglu_quantize_act_1x128(dev_bf16(gu))
    torch.cuda.synchronize()
    q, s = host(xq), host(sa)
    rq, rs, h32 = swiglu.swiglu_quantize_act_1x128(gu)
    rel = np.abs(s.astype(np.float64) - rs) / np.maximum(rs.astype(np.float64), 1e-300)
    assert np.all((rs == 0) == (s == 0)), what
    assert rel.max() <= 2.0 ** -20, f"{what}: scale rel diff {rel.max()}"
    bad = q != rq
    if bad.any():
        scale_rows = rs.T.repeat(128, axis=1)                       # [M][I], tile scale per element
        y = np.abs(h32.astype(np.float64) / np.where(scale_rows == 0, 1.0, scale_rows))
        idx = np.searchsorted(_MID, y)
        lo = np.abs(y - _MID[np.clip(idx - 1, 0, len(_MID) - 1)])
        hi = np.abs(y - _MID[np.clip(idx, 0, len(_MID) - 1)])
        near = np.minimum(lo, hi) <= 2.0 ** -16 * np.maximum(y, 2.0 ** -9)
        dg = e4m3.decode(q[bad]).astype(np.float64)
        dr = e4m3.decode(rq[bad]).astype(np.float64)
        neighbour = np.abs(dg - dr) <= np.maximum(np.abs(dr), np.abs(dg)) * 0.25 + 2.0 ** -9
        assert np.all(near[bad] & neighbour), (
            f"{what}: {np.count_nonzero(bad & ~near)} code mismatches away from a rounding boundary")
        assert bad.sum() <= 1e-3 * bad.size, f"{what}: {bad.sum()} boundary exemptions"
    print(f"[{what}] {bad.sum()} boundary-exempt code differences of {bad.size}; max scale rel diff {rel.max():.2e}",
          flush=True)


def gu_of(g, u):
    return np.concatenate([wl.bf16_bits(np.asarray(g, np.float32)), wl.bf16_bits(np.asarray(u, np.float32))], axis=1)


@pytest.mark.parametrize("M,I,gs,us", [(1, 128, 1.0, 1.0), (37, 256, 3.0, 0.5), (300, 640, 8.0, 20.0),
                                       (513, 128, 0.01, 1e3)])
def test_random(M, I, gs, us):
    rng = np.random.default_rng(M + I)
    check(gu_of(rng.standard_normal((M, I)) * gs, rng.standard_normal((M, I)) * us), f"random {M}x{I}")


def test_extreme_gates():
    rng = np.random.default_rng(5)
    M, I = 64, 384
    g = rng.standard_normal((M, I)) * 4
    u = rng.standard_normal((M, I))
    g[0, :] = -80.0                                   # e^-80: h stays in the FP32 normal range
    g[1, :] = 80.0
    g[2, :] = 0.0
    u[3, :] = 0.0
    g[4, :128] = -60.0; u[4, :128] = 1e-3            # a tile of tiny values
    g[5, 128:256] = 0.0                                # an all-zero tile
    check(gu_of(g, u), "extreme gates")


def test_moe_down_input_full_size():
    """The MoE down-projection input: SiLU(g)*u of 8360 routed rows, I = 2048."""
    rows, offsets = wl.routing()
    M = int(offsets[-1])
    rng = np.random.default_rng(404)
    gu = gu_of(rng.standard_normal((M, 2048)), rng.standard_normal((M, 2048)))
    check(gu, "moe_down input 8360x2048")

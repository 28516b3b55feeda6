"""GPU parity on the large workload: online quantization of X[16384x7168] (heavy-tailed
Student-t, nu = 3) and W[18432x7168], then the block-scaled GEMM with FP32 output, all at
full size in the launch configuration the benchmark times (the GPU quantizers feed the GPU
GEMM).  Against the oracle: all of W's codes and block scales bit-exact; 521 rows of X
(every 32nd row, so eight rows of every 256-row tile, and the tile edges) bit-exact; and C
on those rows x all 18432 columns within the usual bound (the reference is the oracle's
FP64 product of its own codes)."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import quant as oq

from helpers import assert_gemm_within_tol, assert_quant_equal, dev_bf16, host

pytestmark = pytest.mark.gpu


def test_large_pipeline_sampled():
    c = wl.large()
    x, w = c["x"], c["w"][0]
    M, K = x.shape
    N = w.shape[0]
    xq, sa = fq.fp8q_quantize_act_1x128(dev_bf16(x))
    wq, sb = fq.fp8q_quantize_w_128x128(dev_bf16(w))
    out = fq.fp8q_gemm_blockscaled(xq, sa, wq, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()

    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([np.arange(0, M, 32), [1, 127, 128, 255, 256, M // 2 - 1, M - 1],
                                     rng.choice(M, 4, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()

    # quantizers: all of W, the sampled rows of X
    rwq, rsb = oq.quantize_w_128x128(w)
    assert_quant_equal(wq, sb, rwq, rsb, "large weight quant, every block")
    rq, rsa = oq.quantize_act_1x128(x[rows])
    assert_quant_equal(xq[ridx], sa[:, ridx], rq, rsa, "large act quant, sampled rows")

    # GEMM on the sampled rows x every column
    xh = oq.dequant_act(rq, rsa)
    wh = oq.dequant_w(rwq, rsb)
    ref = xh @ wh.T
    got = host(out[ridx]).astype(np.float64)
    assert_gemm_within_tol(got, ref, np.linalg.norm(xh, axis=1), np.linalg.norm(wh, axis=1),
                           f"large 16384x18432x7168 fp32 out, {len(rows)} rows x all columns")

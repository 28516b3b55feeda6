"""GPU parity on the large workload: online quantization of X[16384x7168] (heavy-tailed
Student-t, nu = 3) and W[18432x7168], then the block-scaled GEMM with FP32 output, all at
full size in the launch configuration the benchmark times (the GPU quantizers feed the GPU
GEMM).  Sampled against the oracle: 32 rows of X (codes and scales bit-exact), 8 weight row
blocks of 128 (bit-exact), and C on those 32 rows x the 1024 columns of those blocks
within the usual bound (the reference is the oracle's FP64 product of its own codes)."""
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
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, M // 2 - 1, M // 2, M - 1],
                                     rng.choice(M, 23, replace=False)]))
    blocks = np.unique(np.concatenate([[0, 1, N // 256, N // 128 - 1], rng.choice(N // 128, 4, replace=False)]))

    # quantizers: sampled rows of X, sampled 128-row blocks of W
    rq, rsa = oq.quantize_act_1x128(x[rows])
    assert_quant_equal(xq[torch.from_numpy(rows).cuda()], sa[:, torch.from_numpy(rows).cuda()], rq, rsa,
                       "large act quant, sampled rows")
    wrows = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    rwq, rsb = oq.quantize_w_128x128(w[wrows])
    widx = torch.from_numpy(wrows).cuda()
    assert_quant_equal(wq[widx], sb[torch.from_numpy(blocks).cuda()], rwq, rsb, "large weight quant, sampled blocks")

    # GEMM on the sampled rows x the sampled blocks' columns
    xh = oq.dequant_act(rq, rsa)
    wh = oq.dequant_w(rwq, rsb)
    ref = xh @ wh.T
    got = host(out[torch.from_numpy(rows).cuda()][:, widx]).astype(np.float64)
    assert_gemm_within_tol(got, ref, np.linalg.norm(xh, axis=1), np.linalg.norm(wh, axis=1),
                           "large 16384x18432x7168 fp32 out, sampled")

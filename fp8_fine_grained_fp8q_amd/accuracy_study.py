"""Accuracy of online fine-grained FP8 scaling against the prior-art scalings, on one GPU.

For each workload (the dense projection with 8 outlier channels x100, and the large
Student-t(3) problem) the GEMM C = X W^T is computed through the library three ways and
compared with the FP64 product of the original BF16 operands:

* fine-grained online: 1x128 activation tiles, 128x128 weight blocks (the pages' method);
* tensor-level: one scale per tensor from its current amax;
* delayed: one scale per tensor from an amax history whose maximum is a fraction of the
  current amax (the tensor's range grew since the history was recorded), so the values
  beyond it saturate.

Reported per scheme: relative Frobenius error of C, of the dequantized X and W, the share of
X's values that quantize to zero, and the saturated count.  All quantization and GEMMs run
in the library; torch only supplies memory, the FP64 reference product and the norms.

    python -m fp8_fine_grained_fp8q_amd.accuracy_study [--workloads dense,large] [--out FILE]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import fp8_fine_grained_fp8q_amd as fq  # noqa: E402
import workloads as wl  # noqa: E402


def decode(q: torch.Tensor) -> torch.Tensor:
    return q.view(torch.float8_e4m3fn).to(torch.float64)


def rel(a: torch.Tensor, b: torch.Tensor) -> float:
    return float(torch.linalg.norm(a - b) / torch.linalg.norm(b))


def study(name: str, growth: float):
    cfg = wl.CONFIGS[name]()
    x = torch.from_numpy(cfg["x"].view(np.int16)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(cfg["w"][0].view(np.int16)).view(torch.bfloat16).cuda()
    M, K = x.shape
    N = w.shape[0]
    xd, wd = x.to(torch.float64), w.to(torch.float64)
    c_ref = xd @ wd.T
    out = {"workload": name, "M": M, "N": N, "K": K}

    # fine-grained online
    xq, sa = fq.fp8q_quantize_act_1x128(x)
    wq, sb = fq.fp8q_quantize_w_128x128(w)
    c = fq.fp8q_gemm_blockscaled(xq, sa, wq, sb, out_dtype=torch.float32).to(torch.float64)
    xh = (decode(xq).view(M, K // 128, 128) * sa.T.to(torch.float64)[:, :, None]).view(M, K)
    wh = (decode(wq).view(N // 128, 128, K // 128, 128)
          * sb.to(torch.float64)[:, None, :, None]).view(N, K)
    out["fine_grained"] = {"C_rel_err": rel(c, c_ref), "X_rel_err": rel(xh, xd), "W_rel_err": rel(wh, wd),
                           "X_zero_codes": float(((xq & 0x7F) == 0).double().mean() - (x == 0).double().mean()),
                           "saturated": 0}

    def tensor_scheme(scale_x=None, scale_w=None):
        qx, stx = fq.fp8q_quantize_per_tensor(x, scale_x)
        qw, stw = fq.fp8q_quantize_per_tensor(w, scale_w)
        ax, satx, sx = fq.tensor_stats(stx)
        aw, satw, sw = fq.tensor_stats(stw)
        sa_b = torch.full((K // 128, M), sx, dtype=torch.float32, device="cuda")
        sb_b = torch.full((N // 128, K // 128), sw, dtype=torch.float32, device="cuda")
        cc = fq.fp8q_gemm_blockscaled(qx.view(M, K), sa_b, qw.view(N, K), sb_b,
                                      out_dtype=torch.float32).to(torch.float64)
        return {"C_rel_err": rel(cc, c_ref), "X_rel_err": rel(decode(qx) * sx, xd), "W_rel_err": rel(decode(qw) * sw, wd),
                "X_zero_codes": float(((qx & 0x7F) == 0).double().mean() - (x == 0).double().mean()),
                "saturated": satx + satw, "scale_x": sx, "scale_w": sw}, ax, aw

    out["tensor_level"], ax, aw = tensor_scheme()
    # delayed: the history's largest amax is `growth` times below the current one
    sx_d = torch.tensor([np.float32(np.float32(ax / growth) / np.float32(448.0))], device="cuda")
    sw_d = torch.tensor([np.float32(np.float32(aw / growth) / np.float32(448.0))], device="cuda")
    out["delayed"], _, _ = tensor_scheme(sx_d, sw_d)
    out["delayed"]["history_amax_fraction"] = 1.0 / growth
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", default="dense,large")
    ap.add_argument("--growth", type=float, default=2.0, help="current amax / history amax for delayed scaling")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    fq.load_library()
    res = [study(n, args.growth) for n in args.workloads.split(",")]
    for r in res:
        print(json.dumps(r), flush=True)
    if args.out:
        with open(args.out, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()

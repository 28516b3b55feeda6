"""Build libfp8q.so (gfx950 HIP kernels + the C ABI) in-tree with hipcc.

    python -m fp8_fine_grained_fp8q_amd.build

The library lands next to this file.  Compiles for gfx950 only.  FP32 packed
math (v_pk_*_f32) is disabled in the device code; FP32 denormals stay enabled
(the quantizers rely on IEEE subnormal behaviour) and no fast-math flag is used,
so FP32 division is correctly rounded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8q.so")
SOURCES = ["quant.hip", "gemm.hip", "moe.hip", "fp8q_abi.cpp"]
# Streaming-bandwidth and unit-rate probes the kernels are read against (not part of the path).
PROBE_LIB = os.path.join(HERE, "libfp8q_probe.so")
PROBE_SOURCES = ["stream_probe.hip", "unit_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8q)")


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature; drop that one warning.
    err = "\n".join(line for line in res.stderr.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))

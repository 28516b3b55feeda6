"""The quantizers' division for BF16 dividends (one correction after x * RN(1/s)) is the
correctly rounded quotient for every BF16 significand and every FP32 scale significand:
compiled from `tests/division_exhaustive.c` and run on the host (a few seconds on 8 cores).
The GPU parity tests compare the kernels' codes with the oracle's RN32(x/s) on data; this
covers every significand pair once."""
import shutil
import subprocess
from pathlib import Path

import pytest

SRC = Path(__file__).with_name("division_exhaustive.c")


def test_one_correction_division_is_correctly_rounded(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "division_exhaustive"
    cmd = [gcc, "-O2", "-ffp-contract=off", "-fopenmp", str(SRC), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(res.stdout.strip())
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("0 mismatches in 2147483648 quotients")

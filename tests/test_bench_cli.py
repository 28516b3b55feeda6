"""Host-side checks of the benchmark's command line (no GPU): more than one GPU is refused
with a message, and the documented options parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_options_parse():
    sys.path.insert(0, ROOT)
    import bench
    saved = sys.argv
    try:
        sys.argv = ["bench.py", "--steps", "7", "--warmup", "3", "--settle-ms", "0", "--workload", "moe_layer",
                    "--quant", "separate", "--vendor-context", "--no-cpu-baseline"]
        a = bench.parse()
    finally:
        sys.argv = saved
    assert (a.steps, a.warmup, a.settle_ms, a.workload, a.quant) == (7, 3, 0.0, "moe_layer", "separate")
    assert a.vendor_context and a.no_cpu_baseline and a.gpus == 1
    assert set(bench.WORKLOADS) == {"dense", "large", "moe_up", "moe_down", "moe_ffn", "moe_layer", "train"}

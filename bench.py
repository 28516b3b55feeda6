#!/usr/bin/env python3
"""Benchmark of the FP8 fine-grained quantization + block-scaled GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
    1. online 1x128 activation quantization of X (BF16 -> E4M3 codes + FP32 tile scales)
    2. online 128x128 weight quantization of W (BF16 -> E4M3 codes + FP32 block scales;
       weights change every training step, so they are quantized every step)
    3. block-scaled FP8 GEMM C = X W^T with FP32 promotion every 128 K (BF16 or FP32 out),
       grouped over experts for the MoE workloads.
Steps 1 and 2 run as one launch (fp8q_quantize_act_w) unless --quant separate; either way
each quantizer is also timed in its own launches after the timed steps.
Default workload: the dense projection X[4096x7168] x W[7168x7168]^T, BF16 out.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense|large|moe_up|moe_down|moe_ffn|moe_layer|train]

The `moe_ffn` workload runs the expert FFN forward: activation and expert-weight
quantization, the grouped up-projection, the fused SwiGLU + 1x128 quantizer, and the grouped
down-projection; value = both GEMMs' FLOPs per step.
The `moe_layer` workload runs the whole expert layer from the token side: both quantizers of
X (token order) and W_up in one launch, the expert-parallel dispatch of the codes and scales
to the 32 local experts' rows, the two grouped GEMMs with the fused SwiGLU quantizer and the
W_down quantizer between them, and the gated combine back to the tokens.
The `train` workload runs one training step of the dense layer instead: both-orientation
quantization of X and dY, the transposing weight quantizer, and the three GEMMs (forward,
dgrad through the W^T blocks, wgrad over token tiles); value = 3*2*M*N*K FLOPs per step.

Prints ONE JSON line.  `value` = 2*M*N*K*steps / (timed wall time of the steps), i.e. GEMM
TFLOP/s including both online quantizers.  Inputs are resident in HBM before timing.  To
keep the 256 MB Infinity Cache from serving repeated steps, steps rotate over several
buffer sets (together larger than the cache).

Timing phases: (1) warm-up: the W untimed steps, continued back to back until at least
--settle-ms of them have run, because the GPU's clocks take tens of milliseconds of
sustained load to settle (per-step time falls by about 15 % over the first ~50 ms of
back-to-back steps and then holds); (2) the timed region: exactly K steps launched back to
back, bracketed by a device synchronize and HIP events on the kernels' stream, nothing
recorded between the kernels; (3) the kernel-timing pass: K more steps, identical but with
a HIP event recorded on the kernels' stream between consecutive launches, which gives each
kernel's average launch duration (each event adds a marker between two kernels, which is
why the timed region records none); (4) unless --clock-seconds 0, untimed steps for two more
seconds while amdsmi samples the graphics clock and socket power (its metrics refresh about
once a second), which gives the FP8 peak at the clock the step actually runs at.  `roofline` describes the dominant kernel (the
GEMM): algorithmic FLOPs per launch / its average duration, against the 5.0 PFLOP/s dense
FP8 peak.  `cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "FP8 block-scaled GEMM TFLOP/s incl. online quant; % FP8 MFMA peak; quant GB/s"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_fp8q_amd", "csrc", "gemm.hip")

WORKLOADS = {
    "dense": "dense projection X[4096x7168] . W[7168x7168]^T, bf16 out",
    "large": "large fused pipeline X[16384x7168] (Student-t 3) . W[18432x7168]^T, fp32 out",
    "moe_up": "MoE up-projection, 32 local experts of 256 (top-8 routing of 8192 tokens), W[32][4096x7168], bf16 out",
    "moe_down": "MoE down-projection, 32 local experts, SiLU(g)*u inputs [n x 2048], W[32][7168x2048], bf16 out",
    "moe_ffn": "MoE expert FFN forward, 32 local experts (top-8 routing of 8192 tokens, 8360 rows): "
               "X[8360x7168] -> up W[32][4096x7168] -> SwiGLU+quant -> down W[32][7168x2048], bf16 out",
    "train": "training step of the dense projection X[4096x7168], W[7168x7168]: forward Y = X W^T (bf16), "
             "dgrad dX = dY W (bf16), wgrad dW = dY^T X over the 4096 tokens (fp32)",
    "moe_layer": "MoE expert layer from the token side, one GPU's share: 8192 tokens X[8192x7168] in token order, "
                 "top-8 of 256 routing, 32 local experts: quantize X and W_up -> dispatch (8360 rows) -> up "
                 "W[32][4096x7168] -> SwiGLU+quant -> down W[32][7168x2048] -> gated combine, bf16 out",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="continue the untimed warm-up steps until this many ms of them have run")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="after the timed phases, run untimed steps this long and sample the GPU clock and "
                         "socket power (amdsmi) during the second half; 0 skips it")
    ap.add_argument("--workload", default="dense", choices=sorted(WORKLOADS))
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0: enough to exceed the 256 MB cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quant", choices=("fused", "separate"), default="fused",
                    help="quantize X and W in one launch (fp8q_quantize_act_w) or in two")
    ap.add_argument("--vendor-context", action="store_true",
                    help="also time hipBLASLt's FP8 GEMM (torch._scaled_mm, per-tensor and row-wise scales, "
                         "no per-128-K promotion) on the same shape; reported as vendor_context, not part of "
                         "the step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy per step (untimed) for counter calibration")
    return ap.parse_args()


def gen(workload: str):
    import workloads as wl
    return wl.CONFIGS[workload]()


def source_hash() -> str:
    """The GEMM source's code hash (comments and blank lines removed), the key of the
    committed counter and traffic summaries."""
    from fp8_fine_grained_fp8q_amd.srchash import code_hash
    return code_hash(GEMM_SOURCE)


def measured_traffic(workload: str):
    """HBM bytes per GEMM launch from the committed counter summary, only if it was taken on
    the current GEMM source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != source_hash():
        return None
    return t.get("workloads", {}).get(workload, {}).get("bytes_per_launch")


COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemm_counters.json")


def dense_kernel_name():
    """The dense GEMM kernel the library launches for the benchmarked shapes: the ping-pong
    kernel (256-wide tiles for every shape here), or the split-plan kernel when
    FP8Q_DENSE_KERNEL=split selects it."""
    if os.environ.get("FP8Q_DENSE_KERNEL", "") == "split":
        return "gemm_blockscaled_split_kernel<8, 6, false>"
    return "gemm_pp_kernel<8>"


def measured_counters(kernel_substring: str):
    """Matrix-core busy, vector-ALU busy and LDS figures of the GEMM from the committed
    counter summary (fp8_fine_grained_fp8q_amd/counter_summary.py), only if it was taken on
    the current GEMM source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            entry = json.load(f).get(kernel_substring)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("gemm_source_sha256_16") != source_hash():
        return None
    keys = ("mfma_busy", "valu_busy", "coexec", "lds_bank_conflict", "wait_lds_share", "clock_ghz_from_gui")
    return {k: entry[k] for k in keys if k in entry}


def run_steps(torch, args, step, n_calls):
    """The three timing phases (module docstring) around `step(i, ev)`, which launches step
    i's kernels on the current stream, recording ev[j] before its j-th launch and ev[n_calls]
    after the last one when ev is given.  Returns (wall seconds of the K timed steps, device
    seconds between the timed region's bracketing events, mean microseconds per launch from
    the kernel-timing pass, warm-up steps run)."""
    stream = torch.cuda.current_stream()
    n = 0
    t0 = time.perf_counter()
    while n < args.warmup or (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        step(n, None)
        n += 1
        if n % 10 == 0:  # keeps the host at most 10 steps ahead of the GPU
            torch.cuda.synchronize()
    K_steps = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K_steps):
        step(n + i, None)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_dev = e0.elapsed_time(e1) * 1e-3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)] for _ in range(K_steps)]
    for i in range(K_steps):
        step(n + K_steps + i, evs[i])
    torch.cuda.synchronize()
    samples = [[evs[i][j].elapsed_time(evs[i][j + 1]) * 1e3 for i in range(K_steps)] for j in range(n_calls)]
    per = [float(np.mean(v)) for v in samples]
    args.launch_stats = [{"median": round(float(np.median(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
                          "p90": round(float(np.percentile(v, 90)), 2)} for v in samples]
    args.clock = sustained_clock(torch, args, step, n + 2 * K_steps)
    return wall, t_dev, per, n


def separate_launch_time(torch, stream, src, launch, make_out, n=20):
    """Seconds per launch of one quantizer run alone: n back-to-back launches between two HIP
    events (no marker between them), over enough copies of the input(s) `src` (a tensor or a
    tuple of tensors) and of the outputs that the 256 MB Infinity Cache cannot serve a
    repeated read."""
    src = src if isinstance(src, tuple) else (src,)
    nbytes = sum(t.numel() * t.element_size() for t in src)
    copies = max(2, int(np.ceil(3 * 256e6 / nbytes)))
    srcs = [src] + [tuple(t.clone() for t in src) for _ in range(copies - 1)]
    outs = [make_out() for _ in range(copies)]
    for i in range(copies):
        launch(*srcs[i], outs[i])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        launch(*srcs[i % copies], outs[i % copies])
    e1.record(stream)
    torch.cuda.synchronize()
    del srcs, outs
    return e0.elapsed_time(e1) * 1e-3 / n


def sustained_clock(torch, args, step, first):
    """Median graphics clock (mean over the XCDs) and socket power that amdsmi reports while
    back-to-back steps run, sampled in the second half of --clock-seconds of steps; None when
    skipped, a reason string when amdsmi is unavailable."""
    if args.clock_seconds <= 0:
        return None
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as ex:  # pragma: no cover - depends on the machine
        return f"unavailable: {type(ex).__name__}"
    clocks, power = [], []
    try:
        t0 = time.perf_counter()
        i, last = first, 0.0
        while time.perf_counter() - t0 < args.clock_seconds:
            step(i, None)
            i += 1
            if (i - first) % 10 == 0:
                torch.cuda.synchronize()
                now = time.perf_counter() - t0
                if now > args.clock_seconds / 2 and now - last > 0.1:
                    last = now
                    m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                    per_xcd = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
                    clk = float(np.mean(per_xcd)) if per_xcd else m.get("current_gfxclk")
                    if isinstance(clk, (int, float)):
                        clocks.append(float(clk))
                    if isinstance(m.get("current_socket_power"), (int, float)):
                        power.append(float(m["current_socket_power"]))
        torch.cuda.synchronize()
    finally:
        amdsmi.amdsmi_shut_down()
    if not clocks:
        return "unavailable: no clock samples"
    clk = float(np.median(clocks))
    return {"gfxclk_mhz": round(clk), "socket_power_w": round(float(np.median(power))) if power else None,
            "samples": len(clocks), "fp8_peak_at_clock_tflops": round(PEAK_FP8_TFLOPS * clk / 2400.0, 1)}


def timing_fields(args, wall, t_dev, warm, names):
    """The JSON fields that describe the timing phases, with the median and the 10th / 90th
    percentiles of each kernel's launch durations in the kernel-timing pass."""
    return {"warmup_steps_run": warm, "settle_ms": args.settle_ms,
            "device_ms_per_step": round(t_dev / args.steps * 1e3, 4),
            "kernel_timing": "HIP events between launches in a second pass of K identical steps",
            "kernels_us_median_p10_p90": dict(zip(names, args.launch_stats)),
            "sustained_clock": args.clock}


def at_clock(roofline, clock):
    """Adds the dominant kernel's fraction of the FP8 peak at the sampled sustained clock."""
    if isinstance(clock, dict) and roofline.get("unit") == "TFLOP/s":
        roofline["frac_at_sustained_clock"] = round(roofline["achieved"] / clock["fp8_peak_at_clock_tflops"], 4)
    return roofline


def vendor_context(torch, M, N, K, steps):
    """hipBLASLt's FP8 GEMM on the same shape through torch._scaled_mm (E4M3 operands, BF16
    out; one scale per tensor, then one per row and column): mean microseconds of `steps`
    back-to-back launches after 20 untimed ones.  Context only: neither form applies
    per-128-K block scales.  This library's block-scaled GEMM is timed the same way on the
    same codes (every tile and block scale 1.0; the FP32 promotion still runs every 128 K)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    a = (torch.randn(M, K, device=dev, generator=g) * 50).to(torch.float8_e4m3fn)
    b = (torch.randn(N, K, device=dev, generator=g) * 50).to(torch.float8_e4m3fn)
    one = torch.ones((), device=dev)
    sa, sb = torch.ones(M, 1, device=dev), torch.ones(1, N, device=dev)
    out = {}
    for kind, (x, y) in (("per_tensor", (one, one)), ("rowwise", (sa, sb))):
        try:
            def run():
                return torch._scaled_mm(a, b.t(), scale_a=x, scale_b=y, out_dtype=torch.bfloat16)
            for _ in range(20):
                run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                run()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            out[f"hipblaslt_scaled_mm_{kind}_us"] = round(us, 1)
            out[f"hipblaslt_scaled_mm_{kind}_tflops"] = round(2.0 * M * N * K / us / 1e6, 1)
        except Exception as ex:  # pragma: no cover - depends on the installed torch
            out[f"hipblaslt_scaled_mm_{kind}"] = f"unavailable: {type(ex).__name__}"
    import fp8_fine_grained_fp8q_amd as fq
    xq, wq = a.view(torch.uint8), b.view(torch.uint8)
    s_act = torch.ones(K // 128, M, device=dev)
    s_w = torch.ones(N // 128, K // 128, device=dev)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(20):
        fq.fp8q_gemm_blockscaled(xq, s_act, wq, s_w, out=c, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fq.fp8q_gemm_blockscaled(xq, s_act, wq, s_w, out=c, stream=stream)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    out["fp8q_gemm_blockscaled_same_codes_us"] = round(us, 1)
    out["fp8q_gemm_blockscaled_same_codes_tflops"] = round(2.0 * M * N * K / us / 1e6, 1)
    return out


def hbm_ceiling(torch, stream, sizes):
    """GB/s of two plain streaming kernels (libfp8q_probe.so) at the quantizers' input sizes:
    a 16-byte-per-lane copy, and a read of BF16 words writing one byte per value (the
    quantizers' 2:1 read/write mix, no arithmetic).  20 back-to-back launches rotated over
    copies larger than the Infinity Cache, as for the quantizers' own figures."""
    import ctypes
    path = os.path.join(ROOT, "fp8_fine_grained_fp8q_amd", "libfp8q_probe.so")
    if not os.path.exists(path):
        return "unavailable: libfp8q_probe.so not built"
    lib = ctypes.CDLL(path)
    for f in (lib.probe_copy, lib.probe_read2_write1):
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        f.restype = ctypes.c_int
    out = {}
    for label, nbytes in sizes.items():
        n16 = nbytes // 16
        src = torch.empty(n16 * 16, dtype=torch.uint8, device="cuda").fill_(0x3c)
        for kind, fn, wbytes in (("copy", lib.probe_copy, n16 * 16), ("read2_write1", lib.probe_read2_write1, n16 * 8)):
            def launch(a, d):
                rc = fn(a.data_ptr(), d.data_ptr(), n16, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"probe launch failed ({rc})")
            t = separate_launch_time(torch, stream, src, launch,
                                     lambda: torch.empty(wbytes, dtype=torch.uint8, device="cuda"))
            moved = n16 * 16 + wbytes
            out[f"{label}_{kind}_GBs"] = round(moved / t / 1e9, 1)
        del src
    return out


def cpu_baseline(cfg, flops_step):
    """The oracle as it stands, on a bounded sample of the workload (rank 0 only)."""
    from oracle import gemm as og
    from oracle import quant as oq
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = None
    x, w, offsets = cfg["x"], cfg["w"], cfg["offsets"]
    M, K = x.shape
    G, N, _ = w.shape
    if offsets is None:
        # whole steps (act quant of every row, the weight quantization, the FP64 GEMM),
        # repeated until about 10 s of host work (at most 5 steps)
        reps, t0 = 0, time.perf_counter()
        while reps < 5 and (reps == 0 or time.perf_counter() - t0 < 10.0):
            xq, sa = oq.quantize_act_1x128(x)
            wq, sb = oq.quantize_w_128x128(w[0])
            og.gemm_blockscaled(xq, sa, wq, sb)
            reps += 1
        t3 = time.perf_counter()
        t_step = (t3 - t0) / reps
        sample = (f"the whole step on the oracle ({M} rows: act quant, weight quant, FP64 GEMM against all "
                  f"{N} columns), {reps} step(s)")
    else:
        g = 0
        while offsets[g + 1] == offsets[g]:
            g += 1
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        t0 = time.perf_counter()
        xq, sa = oq.quantize_act_1x128(x[lo:hi])
        t1 = time.perf_counter()
        wq, sb = oq.quantize_w_128x128(w[g])
        t2 = time.perf_counter()
        og.gemm_blockscaled(xq, sa, wq, sb)
        t3 = time.perf_counter()
        rows_scale = M / (hi - lo)
        t_step = (t1 - t0) * rows_scale + (t2 - t1) * G + (t3 - t2) * rows_scale
        sample = (f"oracle on expert {g} ({hi - lo} rows): act quant and GEMM extrapolated x{rows_scale:.3g} "
                  f"to {M} rows, weight quant x{G} experts")
    # cores: the BLAS threads the oracle's FP64 product runs on (its quantizers are
    # single-threaded numpy); the host's CPU count and this process's affinity alongside
    return {"value": flops_step / t_step / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds_measured": round(t3 - t0, 2), "seconds_per_step": round(t_step, 2),
            "blas_threads": int(threads), "host_cpus": os.cpu_count(), "affinity_cpus": affinity}


def run_moe_ffn(args, torch, fq, dev):
    """The `moe_ffn` workload (see the module docstring)."""
    cfg = gen("moe_ffn")
    x_np, wu_np, wd_np, offsets = cfg["x"], cfg["w"], cfg["w_down"], cfg["offsets"]
    M, K = x_np.shape
    G, N1, _ = wu_np.shape
    I = N1 // 2
    flops = 2.0 * M * N1 * K + 2.0 * M * K * I
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wu0 = torch.from_numpy(wu_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wd0 = torch.from_numpy(wd_np.view(np.int16)).view(torch.bfloat16).to(dev)
    off_d = torch.from_numpy(offsets).to(dev)
    per_set = 2 * (x0.numel() + wu0.numel() + wd0.numel()) * 2
    nsets = min(8, args.sets or max(2, int(np.ceil(3 * 256e6 / per_set))))
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    sets = []
    for i in range(nsets):
        sets.append({
            "x": x0 if i == 0 else x0.clone(), "wu": wu0 if i == 0 else wu0.clone(), "wd": wd0 if i == 0 else wd0.clone(),
            "xq": torch.empty((M, K), dtype=u8, device=dev), "sa": torch.empty((K // 128, M), dtype=f32, device=dev),
            "wuq": torch.empty((G, N1, K), dtype=u8, device=dev), "sbu": torch.empty((G, N1 // 128, K // 128), dtype=f32, device=dev),
            "wdq": torch.empty((G, K, I), dtype=u8, device=dev), "sbd": torch.empty((G, K // 128, I // 128), dtype=f32, device=dev),
            "gu": torch.empty((M, N1), dtype=bf, device=dev),
            "hq": torch.empty((M, I), dtype=u8, device=dev), "sh": torch.empty((I // 128, M), dtype=f32, device=dev),
            "y": torch.empty((M, K), dtype=bf, device=dev),
        })
    stream = torch.cuda.current_stream()
    names = ["quant_act(X)", "quant_w(W_up)", "grouped gemm up", "swiglu_quant(h)", "quant_w(W_down)",
             "grouped gemm down"]

    def step(i, ev=None):
        s = sets[i % nsets]
        calls = [
            lambda: fq.fp8q_quantize_act_1x128(s["x"], xq=s["xq"], sa=s["sa"], stream=stream),
            lambda: fq.fp8q_quantize_w_128x128(s["wu"], wq=s["wuq"], sb=s["sbu"], stream=stream),
            lambda: fq.fp8q_grouped_gemm_blockscaled(s["xq"], s["sa"], s["wuq"], s["sbu"], off_d, out=s["gu"],
                                                     stream=stream),
            lambda: fq.fp8q_swiglu_quantize_act_1x128(s["gu"], xq=s["hq"], sa=s["sh"], stream=stream),
            lambda: fq.fp8q_quantize_w_128x128(s["wd"], wq=s["wdq"], sb=s["sbd"], stream=stream),
            lambda: fq.fp8q_grouped_gemm_blockscaled(s["hq"], s["sh"], s["wdq"], s["sbd"], off_d, out=s["y"],
                                                     stream=stream),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record(stream)
            c()
        if ev is not None:
            ev[len(calls)].record(stream)

    wall, t_dev, per_l, warm = run_steps(torch, args, step, len(names))
    per = dict(zip(names, per_l))
    gflops = {"grouped gemm up": 2.0 * M * N1 * K, "grouped gemm down": 2.0 * M * K * I}
    tflops = {n: round(f / (per[n] * 1e-6) / 1e12, 1) for n, f in gflops.items()}
    dom = max(gflops, key=lambda n: per[n])
    h_bytes = M * N1 * 2 + M * I + 4 * M * (I // 128)
    value = flops * args.steps / wall / 1e12
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; shapes and distributions of the workload, no dataset)",
        "config": {"workload": WORKLOADS["moe_ffn"], "M": M, "hidden": K, "intermediate": I, "experts": G,
                   "buffer_sets": nsets},
        **timing_fields(args, wall, t_dev, warm, names),
        "pct_fp8_peak_step": round(value / PEAK_FP8_TFLOPS * 100, 2),
        "kernels_us": {n: round(v, 2) for n, v in per.items()},
        "gemm_tflops": tflops,
        "swiglu_quant_GBs": round(h_bytes / (per["swiglu_quant(h)"] * 1e-6) / 1e9, 1),
        "roofline": at_clock({"bound": "mfma", "achieved": tflops[dom], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops[dom] / PEAK_FP8_TFLOPS, 4), "traffic": None, "kernel": dom,
                     "flop_per_launch": gflops[dom], "avg_launch_us": round(per[dom], 2)}, args.clock),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_moe_layer(args, torch, fq, dev):
    """The `moe_layer` workload (see the module docstring)."""
    cfg = gen("moe_layer")
    x_np, wu_np, wd_np, ids_np, gate_np = cfg["x"], cfg["w"], cfg["w_down"], cfg["topk_ids"], cfg["topk_w"]
    T, K = x_np.shape
    G, N1, _ = wu_np.shape
    I = N1 // 2
    # rows of this batch's dispatch: its routing is an input, so the buffers are sized to it
    R = int(np.count_nonzero((ids_np >= cfg["e_begin"]) & (ids_np < cfg["e_begin"] + G)))
    flops = 2.0 * R * N1 * K + 2.0 * R * K * I
    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wu0 = torch.from_numpy(wu_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wd0 = torch.from_numpy(wd_np.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.from_numpy(ids_np).to(dev)
    gate = torch.from_numpy(gate_np).to(dev)
    per_set = 2 * (x0.numel() + wu0.numel() + wd0.numel()) * 2
    nsets = min(8, args.sets or max(2, int(np.ceil(3 * 256e6 / per_set))))
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    sets = []
    for i in range(nsets):
        sets.append({
            "x": x0 if i == 0 else x0.clone(), "wu": wu0 if i == 0 else wu0.clone(), "wd": wd0 if i == 0 else wd0.clone(),
            "xq": torch.empty((T, K), dtype=u8, device=dev), "sa": torch.empty((K // 128, T), dtype=f32, device=dev),
            "wuq": torch.empty((G, N1, K), dtype=u8, device=dev), "sbu": torch.empty((G, N1 // 128, K // 128), dtype=f32, device=dev),
            "wdq": torch.empty((G, K, I), dtype=u8, device=dev), "sbd": torch.empty((G, K // 128, I // 128), dtype=f32, device=dev),
            "gu": torch.empty((R, N1), dtype=bf, device=dev),
            "hq": torch.empty((R, I), dtype=u8, device=dev), "sh": torch.empty((I // 128, R), dtype=f32, device=dev),
            "out": torch.empty((R, K), dtype=bf, device=dev), "y": torch.empty((T, K), dtype=bf, device=dev),
        })
    stream = torch.cuda.current_stream()
    names = ["quant_act_w(X, W_up)", "dispatch", "grouped gemm up", "swiglu_quant(h)", "quant_w(W_down)",
             "grouped gemm down", "combine"]
    disp = {}

    def step(i, ev=None):
        s = sets[i % nsets]

        def dispatch():
            disp["r"] = fq.fp8q_moe_dispatch(ids, s["xq"], s["sa"], cfg["e_begin"], G, capacity=R, stream=stream)
        calls = [
            lambda: fq.fp8q_quantize_act_w(s["x"], s["wu"], xq=s["xq"], sa=s["sa"], wq=s["wuq"], sb=s["sbu"],
                                           stream=stream),
            dispatch,
            lambda: fq.fp8q_grouped_gemm_blockscaled(disp["r"][0], disp["r"][1], s["wuq"], s["sbu"], disp["r"][2],
                                                     out=s["gu"], stream=stream),
            lambda: fq.fp8q_swiglu_quantize_act_1x128(s["gu"], xq=s["hq"], sa=s["sh"], stream=stream),
            lambda: fq.fp8q_quantize_w_128x128(s["wd"], wq=s["wdq"], sb=s["sbd"], stream=stream),
            lambda: fq.fp8q_grouped_gemm_blockscaled(s["hq"], s["sh"], s["wdq"], s["sbd"], disp["r"][2], out=s["out"],
                                                     stream=stream),
            lambda: fq.fp8q_moe_combine(s["out"], disp["r"][3], gate, y=s["y"], stream=stream),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record(stream)
            c()
        if ev is not None:
            ev[len(calls)].record(stream)

    step(0)
    torch.cuda.synchronize()
    got_rows = int(disp["r"][2][-1].item())
    if got_rows != R:
        raise RuntimeError(f"dispatch produced {got_rows} rows, expected {R}")
    wall, t_dev, per_l, warm = run_steps(torch, args, step, len(names))
    per = dict(zip(names, per_l))
    gflops = {"grouped gemm up": 2.0 * R * N1 * K, "grouped gemm down": 2.0 * R * K * I}
    tflops = {n: round(f / (per[n] * 1e-6) / 1e12, 1) for n, f in gflops.items()}
    dom = max(gflops, key=lambda n: per[n])
    disp_bytes = 2 * (R * K + 4 * R * (K // 128)) + 4 * T * 8 * 2   # codes + scales read and written, maps
    comb_bytes = R * K * 2 + T * K * 2 + 8 * T * 8                  # expert outputs read, y written, maps
    value = flops * args.steps / wall / 1e12
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; shapes and distributions of the workload, no dataset)",
        "config": {"workload": WORKLOADS["moe_layer"], "tokens": T, "rows": R, "hidden": K, "intermediate": I,
                   "experts": G, "buffer_sets": nsets},
        **timing_fields(args, wall, t_dev, warm, names),
        "pct_fp8_peak_step": round(value / PEAK_FP8_TFLOPS * 100, 2),
        "kernels_us": {n: round(v, 2) for n, v in per.items()},
        "gemm_tflops": tflops,
        "dispatch_GBs": round(disp_bytes / (per["dispatch"] * 1e-6) / 1e9, 1),
        "combine_GBs": round(comb_bytes / (per["combine"] * 1e-6) / 1e9, 1),
        "roofline": at_clock({"bound": "mfma", "achieved": tflops[dom], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops[dom] / PEAK_FP8_TFLOPS, 4), "traffic": None, "kernel": dom,
                     "flop_per_launch": gflops[dom], "avg_launch_us": round(per[dom], 2)}, args.clock),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_train(args, torch, fq, dev):
    """The `train` workload (see the module docstring)."""
    cfg = gen("train")
    M, K = cfg["x"].shape
    N = cfg["w"].shape[1]
    flops = 3 * 2.0 * M * N * K
    x0 = torch.from_numpy(cfg["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(cfg["w"][0].view(np.int16)).view(torch.bfloat16).to(dev)
    dy0 = torch.from_numpy(cfg["dy"].view(np.int16)).view(torch.bfloat16).to(dev)
    per_set = 2 * (x0.numel() + w0.numel() + dy0.numel()) * 2 + 4 * N * K
    nsets = min(8, args.sets or max(2, int(np.ceil(3 * 256e6 / per_set))))
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    sets = []
    for i in range(nsets):
        sets.append({
            "x": x0 if i == 0 else x0.clone(), "w": w0 if i == 0 else w0.clone(), "dy": dy0 if i == 0 else dy0.clone(),
            "xq": torch.empty((M, K), dtype=u8, device=dev), "sa": torch.empty((K // 128, M), dtype=f32, device=dev),
            "xqt": torch.empty((K, M), dtype=u8, device=dev), "sat": torch.empty((M // 128, K), dtype=f32, device=dev),
            "wq": torch.empty((N, K), dtype=u8, device=dev), "sb": torch.empty((N // 128, K // 128), dtype=f32, device=dev),
            "wqt": torch.empty((K, N), dtype=u8, device=dev), "sbt": torch.empty((K // 128, N // 128), dtype=f32, device=dev),
            "dyq": torch.empty((M, N), dtype=u8, device=dev), "sdy": torch.empty((N // 128, M), dtype=f32, device=dev),
            "dyqt": torch.empty((N, M), dtype=u8, device=dev), "sdyt": torch.empty((M // 128, N), dtype=f32, device=dev),
            "y": torch.empty((M, N), dtype=bf, device=dev), "dx": torch.empty((M, K), dtype=bf, device=dev),
            "dw": torch.empty((N, K), dtype=f32, device=dev),
        })
    stream = torch.cuda.current_stream()
    names = ["quant_act_dual(X)", "quant_w_t(W)", "gemm fwd", "quant_act_dual(dY)", "gemm dgrad", "gemm_rowscaled wgrad"]

    def step(i, ev=None):
        s = sets[i % nsets]
        calls = [
            lambda: fq.fp8q_quantize_act_dual(s["x"], s["xq"], s["sa"], s["xqt"], s["sat"], stream=stream),
            lambda: fq.fp8q_quantize_w_128x128_t(s["w"], s["wq"], s["sb"], s["wqt"], s["sbt"], stream=stream),
            lambda: fq.fp8q_gemm_blockscaled(s["xq"], s["sa"], s["wq"], s["sb"], out=s["y"], stream=stream),
            lambda: fq.fp8q_quantize_act_dual(s["dy"], s["dyq"], s["sdy"], s["dyqt"], s["sdyt"], stream=stream),
            lambda: fq.fp8q_gemm_blockscaled(s["dyq"], s["sdy"], s["wqt"], s["sbt"], out=s["dx"], stream=stream),
            lambda: fq.fp8q_gemm_rowscaled(s["dyqt"], s["sdyt"], s["xqt"], s["sat"], out=s["dw"], stream=stream),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record(stream)
            c()
        if ev is not None:
            ev[len(calls)].record(stream)

    wall, t_dev, per_l, warm = run_steps(torch, args, step, len(names))
    per = dict(zip(names, per_l))
    gemm_flops = 2.0 * M * N * K
    tflops = {n: round(gemm_flops / (per[n] * 1e-6) / 1e12, 1) for n in names if n.startswith("gemm")}
    dom = max((n for n in names if n.startswith("gemm")), key=lambda n: per[n])
    value = flops * args.steps / wall / 1e12
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; shapes and distributions of the workload, no dataset)",
        "config": {"workload": WORKLOADS["train"], "M": M, "N": N, "K": K, "buffer_sets": nsets},
        **timing_fields(args, wall, t_dev, warm, names),
        "pct_fp8_peak_step": round(value / PEAK_FP8_TFLOPS * 100, 2),
        "kernels_us": {n: round(v, 2) for n, v in per.items()},
        "gemm_tflops": tflops,
        "roofline": at_clock({"bound": "mfma", "achieved": tflops[dom], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops[dom] / PEAK_FP8_TFLOPS, 4), "traffic": None, "kernel": dom,
                     "flop_per_launch": gemm_flops, "avg_launch_us": round(per[dom], 2)}, args.clock),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library is a single-GPU implementation "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_fine_grained_fp8q_amd as fq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fq.load_library()
    dev = torch.device("cuda:0")
    if args.workload in ("train", "moe_ffn", "moe_layer"):
        {"train": run_train, "moe_ffn": run_moe_ffn, "moe_layer": run_moe_layer}[args.workload](args, torch, fq, dev)
        return

    t_gen = time.perf_counter()
    cfg = gen(args.workload)
    x_np, w_np, offsets_np = cfg["x"], cfg["w"], cfg["offsets"]
    M, K = x_np.shape
    G, N, _ = w_np.shape
    grouped = offsets_np is not None
    out_dtype = torch.float32 if cfg["out_dtype"] == "f32" else torch.bfloat16
    print(f"[bench] workload {args.workload}: M={M} N={N} K={K} G={G} generated in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    flops = 2.0 * M * N * K
    bytes_act = 2 * M * K + M * K + 4 * M * (K // 128)
    bytes_w = G * (2 * N * K + N * K + 4 * (N // 128) * (K // 128))
    out_bytes = M * N * (4 if out_dtype == torch.float32 else 2)
    bytes_gemm = M * K + 4 * M * (K // 128) + G * (N * K + 4 * (N // 128) * (K // 128)) + out_bytes

    x0 = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(w_np.view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = w0 if grouped else w0[0]
    off_d = torch.from_numpy(offsets_np).to(dev) if grouped else None
    per_set = 2 * x0.numel() + 2 * w0.numel() + M * K + G * N * K + out_bytes
    nsets = args.sets or max(2, int(np.ceil(3 * 256e6 / per_set)))
    nsets = min(nsets, 8)
    sets = []
    for i in range(nsets):
        xs = x0 if i == 0 else x0.clone()
        ws = w0 if i == 0 else w0.clone()
        sets.append({
            "x": xs, "w": ws,
            "xq": torch.empty((M, K), dtype=torch.uint8, device=dev),
            "sa": torch.empty((K // 128, M), dtype=torch.float32, device=dev),
            "wq": torch.empty(ws.shape, dtype=torch.uint8, device=dev),
            "sb": torch.empty(((G,) if grouped else ()) + (N // 128, K // 128), dtype=torch.float32, device=dev),
            "c": torch.empty((M, N), dtype=out_dtype, device=dev),
        })
    cal_src = cal_dst = None
    if args.copy_calibration:
        cal_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        cal_dst = torch.empty_like(cal_src)

    stream = torch.cuda.current_stream()

    fused = args.quant == "fused"

    def gemm(s):
        if grouped:
            fq.fp8q_grouped_gemm_blockscaled(s["xq"], s["sa"], s["wq"], s["sb"], off_d, out=s["c"], stream=stream)
        else:
            fq.fp8q_gemm_blockscaled(s["xq"], s["sa"], s["wq"], s["sb"], out=s["c"], stream=stream)

    def step(i, ev=None):
        s = sets[i % nsets]
        if fused:
            calls = [lambda: fq.fp8q_quantize_act_w(s["x"], s["w"], xq=s["xq"], sa=s["sa"], wq=s["wq"], sb=s["sb"],
                                                    stream=stream)]
        else:
            calls = [lambda: fq.fp8q_quantize_act_1x128(s["x"], xq=s["xq"], sa=s["sa"], stream=stream),
                     lambda: fq.fp8q_quantize_w_128x128(s["w"], wq=s["wq"], sb=s["sb"], stream=stream)]
        calls.append(lambda: gemm(s))
        for j, c in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            c()
        if ev is not None:
            ev[len(calls)].record(stream)
        if cal_src is not None and ev is None and i < args.warmup:
            cal_dst.copy_(cal_src)  # counter calibration: a plain copy right after a GEMM

    wall, t_dev, per, warm = run_steps(torch, args, step, 2 if fused else 3)
    K_steps = args.steps
    if cal_src is not None:
        for _ in range(3):
            cal_dst.copy_(cal_src)
        torch.cuda.synchronize()

    # After the timed phases: each quantizer in its own launches, for the per-quantizer
    # figures (in fused mode the timed steps run them as one launch).
    s_act = separate_launch_time(torch, stream, sets[0]["x"], lambda src, d: fq.fp8q_quantize_act_1x128(
        src, xq=d[0], sa=d[1], stream=stream), lambda: (torch.empty_like(sets[0]["xq"]), torch.empty_like(sets[0]["sa"])))
    s_w = separate_launch_time(torch, stream, sets[0]["w"], lambda src, d: fq.fp8q_quantize_w_128x128(
        src, wq=d[0], sb=d[1], stream=stream), lambda: (torch.empty_like(sets[0]["wq"]), torch.empty_like(sets[0]["sb"])))
    s_fused = separate_launch_time(
        torch, stream, (sets[0]["x"], sets[0]["w"]),
        lambda x, w, d: fq.fp8q_quantize_act_w(x, w, xq=d[0], sa=d[1], wq=d[2], sb=d[3], stream=stream),
        lambda: tuple(torch.empty_like(sets[0][k]) for k in ("xq", "sa", "wq", "sb")))

    ceiling = hbm_ceiling(torch, stream, {"x_bf16": 2 * M * K, "w_bf16": 2 * G * N * K})

    ms_per_step = wall / K_steps * 1e3
    value = flops * K_steps / wall / 1e12

    # per-launch means (microseconds) from the kernel-timing pass, in seconds
    a_act, a_w, a_g = (per[0] * 1e-6, 0.0, per[1] * 1e-6) if fused else (per[0] * 1e-6, per[1] * 1e-6, per[2] * 1e-6)
    gemm_tflops = flops / a_g / 1e12
    traffic = measured_traffic(args.workload)
    hbm_gbs = bytes_gemm / a_g / 1e9
    # the binding roof is the one whose time at peak is longer: MFMA for the dense shapes,
    # HBM for the expert GEMMs (each expert's weights are read for a few hundred rows)
    hbm_bound = bytes_gemm / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_FP8_TFLOPS * 1e12)
    kernel = "gemm_grouped_kernel" if grouped else dense_kernel_name()
    if hbm_bound:
        roofline = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(hbm_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "mfma_achieved_TFLOPs": round(gemm_tflops, 1),
                    "mfma_frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                    "hbm_achieved_GBs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}
    roofline.update({"kernel": kernel, "flop_per_launch": flops, "avg_launch_us": round(a_g * 1e6, 2),
                     "algorithmic_bytes_per_launch": bytes_gemm})
    counters = measured_counters("gemm_grouped_kernel" if grouped else "gemm_pp")
    if counters:
        roofline["counters"] = counters

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; shapes and distributions of the workload, no dataset)",
        "config": {"workload": WORKLOADS[args.workload], "M": M, "N": N, "K": K, "experts": G,
                   "out": cfg["out_dtype"], "buffer_sets": nsets},
        **timing_fields(args, wall, t_dev, warm,
                        (["quantize_act_w (fused)"] if fused else ["quantize_act_1x128", "quantize_w_128x128"])
                        + ["gemm"]),
        "pct_fp8_peak_step": round(value / PEAK_FP8_TFLOPS * 100, 2),
        "gemm_only_tflops": round(gemm_tflops, 1),
        # act quant (its own launch) + GEMM only, the weights quantized in a separate call
        "act_quant_plus_gemm_tflops": round(flops / (s_act + a_g) / 1e12, 1),
        "quant": args.quant,
        "kernels_us": ({"quantize_act_w (fused)": round(a_act * 1e6, 2)} if fused else
                       {"quantize_act_1x128": round(a_act * 1e6, 2), "quantize_w_128x128": round(a_w * 1e6, 2)})
        | {"gemm": round(a_g * 1e6, 2),
           "own launches, back to back: quantize_act_1x128": round(s_act * 1e6, 2),
           "own launches, back to back: quantize_w_128x128": round(s_w * 1e6, 2),
           "own launches, back to back: quantize_act_w": round(s_fused * 1e6, 2)},
        # act_w: the quantizer launch of the steps (kernel-timing pass; fused mode only);
        # *_own: each quantizer alone, back-to-back launches with no event marker between
        # them, inputs rotated past the Infinity Cache
        "quant_GBs": ({"act_w": round((bytes_act + bytes_w) / a_act / 1e9, 1),
                       "act_w_frac_hbm": round((bytes_act + bytes_w) / a_act / 1e9 / PEAK_HBM_GBS, 4)} if fused else {})
        | {"act_w_own": round((bytes_act + bytes_w) / s_fused / 1e9, 1),
           "act_w_own_frac_hbm": round((bytes_act + bytes_w) / s_fused / 1e9 / PEAK_HBM_GBS, 4),
           "act": round(bytes_act / s_act / 1e9, 1), "act_frac_hbm": round(bytes_act / s_act / 1e9 / PEAK_HBM_GBS, 4),
           "w": round(bytes_w / s_w / 1e9, 1), "w_frac_hbm": round(bytes_w / s_w / 1e9 / PEAK_HBM_GBS, 4)},
        # what plain streaming kernels of the same sizes reach on this device (achievable ceiling)
        "hbm_ceiling": ceiling,
        "roofline": at_clock(roofline, args.clock),
        "cpu_baseline": None,
    }
    if args.vendor_context and not grouped:
        line["vendor_context"] = vendor_context(torch, M, N, K, K_steps)
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        line["cpu_baseline"] = cpu_baseline(cfg, flops)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

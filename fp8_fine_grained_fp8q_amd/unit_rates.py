"""Unit rates of one CU on the device: LDS reads, direct-to-LDS copies from L2, and the
matrix core with and without the GEMM's FP32 promotion FMAs (the probes of
csrc/unit_probe.hip, in libfp8q_probe.so).

    python -m fp8_fine_grained_fp8q_amd.unit_rates [--json PATH]

One workgroup of 8 waves per CU, one launch per probe after a warm-up launch; per
workgroup the shader-clock cycles (s_memtime) and the 100 MHz reference ticks
(s_memrealtime) of the timed loop give bytes or busy cycles per clock and the clock.
Medians over the workgroups are printed.  Measurement infrastructure only: no part of the
quantization or GEMM path.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "libfp8q_probe.so")
THREADS = 512
MFMA_BUSY_CYCLES = 32  # v_mfma_f32_16x16x128_f8f6f4


def _lib():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} not built (python -m fp8_fine_grained_fp8q_amd.build)")
    lib = ctypes.CDLL(PROBE_LIB)
    for f in (lib.probe_lds_read, lib.probe_lds_copy, lib.probe_lds_mix, lib.probe_mfma):
        f.restype = ctypes.c_int
    return lib


def _median(t: torch.Tensor) -> float:
    return float(t.median())


def run() -> dict:
    lib = _lib()
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(blocks * THREADS, dtype=torch.int32, device=dev)
    cyc = torch.zeros(4 * blocks, dtype=torch.int64, device=dev)
    src = torch.randint(0, 256, (512 * 1024,), dtype=torch.uint8, device=dev,
                        generator=torch.Generator(device=dev).manual_seed(5))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p_out, p_cyc = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(cyc.data_ptr())

    def timed(call):
        for _ in range(2):  # warm-up launch, then the measured one
            rc = call()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
            torch.cuda.synchronize()
        c = cyc[: 2 * blocks].cpu().view(blocks, 2).double()
        return c[:, 0], c[:, 1] * 10.0  # cycles, ns

    res = {"cus": blocks, "waves_per_cu": THREADS // 64}
    iters = 4096
    cy, ns = timed(lambda: lib.probe_lds_read(blocks, iters, p_out, p_cyc, stream))
    byts = (THREADS // 64) * iters * 8 * 1024
    res["lds_read_b128"] = {"bytes_per_clk_cu": round(_median(byts / cy), 1), "ghz": round(_median(cy / ns), 3)}
    for mode, name, per in ((0, "lds_copy_16B_per_lane", 1024), (1, "lds_copy_4B_per_lane", 256),
                            (2, "load_16B_per_lane_to_vgprs", 1024)):
        iters = 2000
        cy, ns = timed(lambda: lib.probe_lds_copy(mode, blocks, iters, ctypes.c_void_p(src.data_ptr()), p_out,
                                                  p_cyc, stream))
        byts = (THREADS // 64) * iters * 8 * per
        res[name] = {"bytes_per_clk_cu": round(_median(byts / cy), 1),
                     "GBs_per_cu": round(_median(byts / ns), 1),
                     "TBs_chip": round(_median(byts / ns) * blocks / 1000, 2),
                     "ghz": round(_median(cy / ns), 3)}
    # 4 waves reading LDS (bursts of 8 or 16 one-KB reads, each waited for) beside 4 waves
    # copying into it, each half alone and both together
    ic = 1800
    cases = [(8, "lds_read_4_waves_burst8_alone", 8192, 0), (16, "lds_read_4_waves_burst16_alone", 4096, 0),
             (8, "lds_copy_4_waves_alone", 0, ic), (8, "lds_read_burst8_and_copy_together", 8192, ic),
             (16, "lds_read_burst16_and_copy_together", 4096, ic)]
    for burst, name, a, b in cases:
        for _ in range(2):
            rc = lib.probe_lds_mix(burst, blocks, a, b, ctypes.c_void_p(src.data_ptr()), p_out, p_cyc, stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
            torch.cuda.synchronize()
        c = cyc.cpu().view(blocks, 4).double()
        entry = {}
        if a:
            entry["read_bytes_per_clk_cu"] = round(_median(4 * a * burst * 1024 / c[:, 0]), 1)
        if b:
            entry["copy_bytes_per_clk_cu"] = round(_median(4 * b * 8 * 1024 / c[:, 2]), 1)
        entry["ghz"] = round(_median(c[:, 0 if a else 2] / (c[:, 1 if a else 3] * 10.0)), 3)
        res[name] = entry
    names = {0: "mfma_chained", 1: "mfma_plus_4_independent_fma", 2: "mfma_promotion_one_column_behind",
             3: "mfma_promotion_at_once", 4: "mfma_promotion_one_column_behind_interleaved"}
    for mode in (0, 1, 2, 3, 4):
        for iters in ((20000, 200000) if mode <= 1 else (10000, 100000)):
            cy, ns = timed(lambda: lib.probe_mfma(mode, blocks, iters, p_out, p_cyc, stream))
            per_iter = 8 if mode <= 1 else 16  # MFMAs per wave and iteration
            busy = (THREADS // 256) * per_iter * iters * MFMA_BUSY_CYCLES / cy
            flop = blocks * (THREADS // 64) * per_iter * iters * 16 * 16 * 128 * 2
            run_len = "short" if iters in (20000, 10000) else "long"
            res[f"{names[mode]}_{run_len}"] = {"mfma_busy": round(_median(busy), 3), "ghz": round(_median(cy / ns), 3),
                                               "TFLOPs": round(flop / float(ns.max()) / 1e3, 0),
                                               "ms": round(float(ns.max()) / 1e6, 2)}
    return res


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--json", help="also write the figures to this file")
    args = ap.parse_args()
    res = run()
    print(json.dumps(res), flush=True)
    for k, v in res.items():
        if isinstance(v, dict):
            print(f"{k:34s} " + ", ".join(f"{a} {b}" for a, b in v.items()), flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()

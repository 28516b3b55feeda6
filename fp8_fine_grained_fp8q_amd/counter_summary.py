"""Summarise rocprofv3 `--pmc` passes (each its own run, with `--kernel-trace`) into
per-kernel counter figures: matrix-core (MFMA) busy fraction, vector-ALU busy fraction,
MFMA/VALU co-issue, LDS bank-conflict and LDS-wait shares, next to the kernel's duration
in the same run.

    python -m fp8_fine_grained_fp8q_amd.counter_summary OUT.json KERNEL_SUBSTR PASS_DIR [PASS_DIR ...]

Each PASS_DIR holds one run's `*_counter_collection.csv` and `*_kernel_trace.csv`.  For the
dispatches whose kernel name contains KERNEL_SUBSTR the counters are averaged per dispatch.
Definitions (SIMD_NUM = 4 per CU; GRBM_GUI_ACTIVE is read per dispatch and normalised by the
number of XCD instances it is summed over, found from its ratio to the traced duration):
  mfma_busy      = sum SQ_VALU_MFMA_BUSY_CYCLES / (SIMD_NUM * CUs * gui_cycles)
  valu_busy      = sum SQ_ACTIVE_INST_VALU * 4 / (SIMD_NUM * CUs * gui_cycles)   (quad-cycle units)
  coexec         = sum SQ_VALU_MFMA_COEXEC_CYCLES / (SIMD_NUM * CUs * gui_cycles)
  lds_bank_conflict = sum SQ_LDS_BANK_CONFLICT / (CUs * gui_cycles)
  wait_lds_share = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES ; wait_any_share = SQ_WAIT_ANY / SQ_WAVE_CYCLES
The GEMM source's code hash (fp8_fine_grained_fp8q_amd/srchash.py: comments and blank
lines removed) is stored so that the benchmark reports these only while the kernel code is
unchanged.
"""
import csv
import glob
import json
import os
import sys

from fp8_fine_grained_fp8q_amd.srchash import code_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_fp8q_amd", "csrc", "gemm.hip")
CUS = 256
SIMDS = 4


def read_pass(d, substr):
    """({counter: mean per matching dispatch}, mean traced duration in ns, dispatches)."""
    cc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    kt = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not cc:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for r in csv.DictReader(open(cc[0])):
        if substr not in r["Kernel_Name"]:
            continue
        key = (int(r["Dispatch_Id"]), r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    disp = sorted({k[0] for k in per})
    counters = {}
    for (dsp, name), v in per.items():
        counters.setdefault(name, []).append(v)
    means = {n: sum(v) / len(v) for n, v in counters.items()}
    dur = None
    if kt:
        ds = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in csv.DictReader(open(kt[0]))
              if substr in r["Kernel_Name"]]
        dur = sum(ds) / len(ds) if ds else None
    return means, dur, len(disp)


def main():
    out, substr, dirs = sys.argv[1], sys.argv[2], sys.argv[3:]
    c, durs, nd = {}, [], []
    for d in dirs:
        m, dur, n = read_pass(d, substr)
        c.update(m)
        nd.append(n)
        if dur:
            durs.append(dur)
    dur_ns = sum(durs) / len(durs) if durs else None
    res = {"kernel_substring": substr, "dispatches_per_pass": nd, "duration_ns_mean": dur_ns,
           "counters_mean_per_dispatch": {k: round(v, 1) for k, v in sorted(c.items())}}
    gui = c.get("GRBM_GUI_ACTIVE")
    if gui and dur_ns:
        # GUI-active cycles per ns is the clock in GHz; a sum over instances reads a multiple
        # (the clock lies in 0.5 .. 2.5 GHz, so one instance or eight XCDs are told apart)
        inst = 8 if gui / dur_ns > 5.0 else 1
        cyc = gui / inst
        res["grbm_instances"] = inst
        res["gui_cycles"] = round(cyc)
        res["clock_ghz_from_gui"] = round(cyc / dur_ns, 3)
        slots = SIMDS * CUS * cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            res["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / slots, 4)
        if "SQ_ACTIVE_INST_VALU" in c:
            res["valu_busy"] = round(c["SQ_ACTIVE_INST_VALU"] * 4 / slots, 4)
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
            res["coexec"] = round(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / slots, 4)
        if "SQ_LDS_BANK_CONFLICT" in c:
            res["lds_bank_conflict"] = round(c["SQ_LDS_BANK_CONFLICT"] / (CUS * cyc), 4)
    if c.get("SQ_WAVE_CYCLES"):
        for k, name in (("SQ_WAIT_INST_LDS", "wait_lds_share"), ("SQ_WAIT_ANY", "wait_any_share"),
                        ("SQ_ACTIVE_INST_LDS", "active_lds_share")):
            if k in c:
                res[name] = round(c[k] / c["SQ_WAVE_CYCLES"], 4)
    res["gemm_source_sha256_16"] = code_hash(GEMM_SOURCE)
    try:
        data = json.load(open(out))
    except (OSError, ValueError):
        data = {}
    data[substr] = res
    with open(out, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()

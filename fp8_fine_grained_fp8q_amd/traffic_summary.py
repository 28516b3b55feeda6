"""Summarise two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) of `bench.py
--copy-calibration` into profiles/gemm_traffic.json and a text table.

Each counter is read in KiB per dispatch.  The bench run also launches a plain device copy
of 256 MiB after each step's GEMM; the ratio between the counter it reports and the bytes it
must move (256 MiB read, 256 MiB written) is the calibration factor applied to the GEMM's
reading.  The calibration copies are the copy dispatches that directly follow a GEMM
dispatch (other copies in the run are input uploads and buffer clones of other sizes).

    python -m fp8_fine_grained_fp8q_amd.traffic_summary WORKLOAD FETCH_CSV WRITE_CSV
"""
import csv
import json
import os
import sys

from fp8_fine_grained_fp8q_amd.srchash import code_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_fp8q_amd", "csrc", "gemm.hip")
OUT = os.path.join(ROOT, "profiles", "gemm_traffic.json")
COPY_BYTES = 256 << 20


def dispatches(path, counter):
    """[(dispatch id, kernel name, counter value in KiB)] in dispatch order."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = acc.get(d, (r["Kernel_Name"], 0.0))
        acc[d] = (name, v + float(r["Counter_Value"]))
    return [(d, n, v) for d, (n, v) in sorted(acc.items())]


def gemm_and_copy(rows):
    """Mean counter of the GEMM dispatches and median of the calibration copies."""
    gemm = [v for _, n, v in rows if "fp8q::gemm_" in n]
    cal = [v for i, (_, n, v) in enumerate(rows)
           if i > 0 and "copy" in n.lower() and "fp8q::gemm_" in rows[i - 1][1]]
    if not gemm or not cal:
        raise SystemExit("no GEMM dispatch or no calibration copy in the counter file")
    cal.sort()
    name = next(n for _, n, _ in rows if "fp8q::gemm_" in n)
    return name, sum(gemm) / len(gemm), cal[len(cal) // 2]


def main():
    workload, fetch_csv, write_csv = sys.argv[1:4]
    name, g_fetch, copy_fetch = gemm_and_copy(dispatches(fetch_csv, "FETCH_SIZE"))
    _, g_write, copy_write = gemm_and_copy(dispatches(write_csv, "WRITE_SIZE"))
    f_fetch = COPY_BYTES / (copy_fetch * 1024.0)
    f_write = COPY_BYTES / (copy_write * 1024.0)
    rd = g_fetch * 1024.0 * f_fetch
    wr = g_write * 1024.0 * f_write
    entry = {
        "kernel": name.split("(")[0],
        "fetch_kib_raw": round(g_fetch, 1), "write_kib_raw": round(g_write, 1),
        "copy_fetch_kib_raw": round(copy_fetch, 1), "copy_write_kib_raw": round(copy_write, 1),
        "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4),
        "read_bytes_per_launch": round(rd), "write_bytes_per_launch": round(wr),
        "bytes_per_launch": round(rd + wr),
    }
    sha = code_hash(GEMM_SOURCE)
    try:
        data = json.load(open(OUT))
    except (OSError, ValueError):
        data = {}
    if data.get("gemm_source_sha256_16") != sha:
        data = {"gemm_source_sha256_16": sha, "workloads": {}}
    data["workloads"][workload] = entry
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps({workload: entry}))


if __name__ == "__main__":
    main()

"""Summarise a rocprofv3 run of bench.py into profiles/: per-kernel durations from the kernel-trace
stats, HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE counter passes calibrated against a
device copy of known size in the same run, and a JSON record that bench.py reads for its roofline
`traffic` field (valid while kernels.hip is unchanged).

Usage: python -m latent_width_expert_amd.profile_summary RUN_DIR WORKLOAD "COMMAND" [TITLE]
RUN_DIR holds kt/kt_kernel_stats.csv (rocprofv3 --kernel-trace --stats -d RUN_DIR/kt -o kt ...),
fetch/fetch_counter_collection.csv and write/write_counter_collection.csv (rocprofv3 --pmc FETCH_SIZE
and --pmc WRITE_SIZE with --kernel-trace, bench flag --calib-copy-mb 1024).
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
STAGE = {0: "x_gemm", 1: "gateup", 2: "down", 3: "y_gemm"}
CALIB_BYTES = 1 << 30


def stage_of(name: str):
    if any(k in name for k in ("panel_gemm_kernel", "tiled_gemm_kernel", "skinny_gemm_kernel", "skinny_reduce_kernel")):
        tag = int(name.split(">(")[0].replace("<", ",").split(",")[-1])
        return STAGE[tag] + (" (reduce)" if "skinny_reduce" in name else "")
    if "tile_items" in name:
        return "gateup/down (item list)"
    for s in ("topk", "route", "combine", "pack", "f32_to_bf16"):
        if s in name:
            return s
    return None


def counters(path):
    rows = list(csv.DictReader(open(path)))
    per = collections.defaultdict(list)
    calib = None
    for r in rows:
        if "copyBuffer" in r["Kernel_Name"]:
            # the calibration copy (the bench's only large device copy)
            v = float(r["Counter_Value"])
            calib = v if calib is None else max(calib, v)
            continue
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}, calib


def main():
    run, workload, cmd = sys.argv[1:4]
    title = sys.argv[4] if len(sys.argv) > 4 else f"Kernel profile: {workload}"
    kern = list(csv.DictReader(open(os.path.join(run, "kt", "kt_kernel_stats.csv"))))
    fetch, cf = counters(os.path.join(run, "fetch", "fetch_counter_collection.csv"))
    write, cw = counters(os.path.join(run, "write", "write_counter_collection.csv"))
    ff = CALIB_BYTES / 1024.0 / cf
    fw = CALIB_BYTES / 1024.0 / cw
    lines = [f"# {title}", "", "Kernel trace:", "", "```", cmd, "```", "",
             "Counter passes: the same bench under `rocprofv3 --pmc FETCH_SIZE --kernel-trace` and "
             "`rocprofv3 --pmc WRITE_SIZE --kernel-trace` with `--steps 3 --warmup 1 --no-cpu-baseline "
             "--calib-copy-mb 1024`; summarised by `python -m latent_width_expert_amd.profile_summary`.", "",
             f"Calibration: the 1 GiB device copy in the same run reads FETCH_SIZE = {cf:.0f} KiB and "
             f"WRITE_SIZE = {cw:.0f} KiB, so FETCH_SIZE is scaled by {ff:.4f} and WRITE_SIZE by {fw:.4f}.", "",
             "| kernel | stage | calls | avg us | FETCH KiB/dispatch | WRITE KiB/dispatch | HBM bytes/dispatch (calibrated) |",
             "|---|---|---|---|---|---|---|"]
    rec = {"kernels_hip_sha256": hashlib.sha256(open(os.path.join(HERE, "csrc", "kernels.hip"), "rb").read()).hexdigest(),
           "fetch_scale": ff, "write_scale": fw, "kernels": {}}
    for r in kern:
        n = r["Name"]
        st = stage_of(n)
        fk, wk = fetch.get(n), write.get(n)
        tb = (fk * ff + wk * fw) * 1024 if fk is not None and wk is not None else None
        lines.append(f"| `{n[:78]}` | {st or ''} | {r['Calls']} | {float(r['AverageNs']) / 1000:.1f} | "
                     f"{'' if fk is None else f'{fk:.0f}'} | {'' if wk is None else f'{wk:.0f}'} | "
                     f"{'' if tb is None else f'{tb:.4g}'} |")
        if st and st not in ("pack",) and tb is not None:
            rec["kernels"][st] = {"symbol": n, "avg_us": float(r["AverageNs"]) / 1000, "fetch_kib": fk,
                                  "write_kib": wk, "hbm_bytes_per_launch": tb}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    open(os.path.join(ROOT, "profiles", f"kernels_{workload}.md"), "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w"), indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()

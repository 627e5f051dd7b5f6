"""Summarise rocprofv3 runs of bench.py into profiles/: per-kernel durations from the kernel trace,
HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE counter passes calibrated against a device copy of
known size in the same run, on-chip counters from further passes, and a JSON record that bench.py
reads for its roofline `traffic` field (valid while kernels.hip is unchanged).

Usage: python -m latent_width_expert_amd.profile_summary RUN_DIR WORKLOAD "COMMANDS" [TITLE]

RUN_DIR holds
  kt/kt_kernel_trace.csv            rocprofv3 --kernel-trace --stats -d RUN_DIR/kt -o kt -- <bench>
  fetch/fetch_counter_collection.csv  rocprofv3 --pmc FETCH_SIZE --kernel-trace ... (bench with
  write/write_counter_collection.csv  --calib-copy-mb 1024), and --pmc WRITE_SIZE likewise
  c*/c*_counter_collection.csv      optional further --pmc passes (SQ_, TA_, TD_, TCP_, TCC_ counters)

Dispatches are grouped by kernel symbol, grid size and bench phase (a new phase starts where weights
are packed after a layer stage has run: each workload a bench run times after the decode batch packs
its own), so the same kernel at the same grid in two workloads yields two rows.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
STAGE = {0: "x_gemm", 1: "gateup", 2: "down", 3: "y_gemm"}
CALIB_BYTES = 1 << 30
N_XCD, N_CU = 8, 256


def stage_of(name: str):
    if any(k in name for k in ("panel_gemm_kernel", "panel_rows_kernel", "tiled_gemm_kernel", "tiled_f8_kernel",
                               "skinny_gemm_kernel", "skinny_reduce_kernel")):
        tag = int(name.split(">(")[0].replace("<", ",").split(",")[-1])
        return STAGE[tag] + (" (reduce)" if "skinny_reduce" in name else "")
    if "tile_items" in name:
        return "gateup/down (item list)"
    if "lora_a" in name:
        return "gateup/down (LoRA first factor)"
    for s in ("topk", "route", "combine", "pack", "f32_to_bf16", "stream_read", "quantile_bias", "gather_rows",
              "send_counts", "offsets_clamped", "fill_i32"):
        if s in name:
            return s
    return None


def phases(rows, name_of, order_of):
    """Phase of each row in dispatch order: 0 up to the first weight packing that follows a layer stage's
    kernel, then one more at each such packing (a workload's weights are packed before its steps)."""
    ph, staged, out = 0, False, []
    for r in sorted(rows, key=order_of):
        name = name_of(r)
        if "pack_kernel" in name and staged:
            ph += 1
            staged = False
        elif stage_of(name) not in (None, "pack"):
            staged = True
        out.append((r, ph))
    return out


def trace(path):
    """(symbol, grid, phase) -> list of durations (ns) from a kernel-trace CSV."""
    per = collections.defaultdict(list)
    rows = list(csv.DictReader(open(path)))
    for r, ph in phases(rows, lambda r: r["Kernel_Name"], lambda r: int(r["Start_Timestamp"])):
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        per[(r["Kernel_Name"], g, ph)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per


def counter_passes(path):
    """(symbol, grid, phase) -> {counter: mean value per dispatch}, and the calibration copy's values."""
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(lambda: collections.defaultdict(set))
    calib = {}
    rows = list(csv.DictReader(open(path)))
    # phases over dispatches (a dispatch has one row per counter)
    first = {}
    for r in rows:
        first.setdefault(int(r["Dispatch_Id"]), r["Kernel_Name"])
    ph_of = {d: ph for (d, _), ph in phases(list(first.items()), lambda dn: dn[1], lambda dn: dn[0])}
    for r in rows:
        name, c, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
        if "copyBuffer" in name:
            # the calibration copy (the bench's only large device copy)
            calib[c] = max(calib.get(c, 0.0), v)
            continue
        key = (name, int(r["Grid_Size"]), ph_of[int(r["Dispatch_Id"])])
        acc[key][c] += v
        disp[key][c].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k][c]) for c, v in d.items()} for k, d in acc.items()}, calib


def derived(c, dur_ns):
    """Ratios of one dispatch's counters. GRBM_GUI_ACTIVE is summed over the XCDs, the MFMA busy
    count over the SIMDs (4 per CU), SQ_BUSY_CYCLES over the shader engines."""
    out = {}
    if "GRBM_GUI_ACTIVE" in c and dur_ns:
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
        out["clock GHz"] = cyc / dur_ns
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            out["MFMA busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_CU * 4)
    if c.get("SQ_WAVE_CYCLES"):
        for k, lab in (("SQ_WAIT_INST_ANY", "wave cycles waiting on a dependency"),
                       ("SQ_ACTIVE_INST_ANY", "wave cycles issuing")):
            if k in c:
                out[lab] = c[k] / c["SQ_WAVE_CYCLES"]
    if c.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in c:
        out["LDS bank-conflict cycles / LDS active"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
    if c.get("TCP_TCC_READ_REQ") and "TCP_TCC_READ_REQ_LATENCY" in c:
        out["L2 read latency (cycles per request)"] = c["TCP_TCC_READ_REQ_LATENCY"] / c["TCP_TCC_READ_REQ"]
    if "TCC_HIT" in c and "TCC_MISS" in c and c["TCC_HIT"] + c["TCC_MISS"] > 0:
        out["L2 hit rate"] = c["TCC_HIT"] / (c["TCC_HIT"] + c["TCC_MISS"])
    if "GRBM_GUI_ACTIVE" in c:
        cyc_cu = c["GRBM_GUI_ACTIVE"] / N_XCD * N_CU
        for k, lab in (("TA_TA_BUSY", "TA busy (per CU)"), ("TD_TD_BUSY", "TD busy (per CU)"),
                       ("TCP_PENDING_STALL_CYCLES", "L1 pending-stall cycles (per CU)")):
            if k in c:
                out[lab] = c[k] / cyc_cu
    return out


def main():
    run, workload, cmd = sys.argv[1:4]
    title = sys.argv[4] if len(sys.argv) > 4 else f"Kernel profile: {workload}"
    kern = trace(os.path.join(run, "kt", "kt_kernel_trace.csv"))
    fetch, cf = counter_passes(os.path.join(run, "fetch", "fetch_counter_collection.csv"))
    write, cw = counter_passes(os.path.join(run, "write", "write_counter_collection.csv"))
    ff = CALIB_BYTES / 1024.0 / cf["FETCH_SIZE"]
    fw = CALIB_BYTES / 1024.0 / cw["WRITE_SIZE"]
    lines = [f"# {title}", "", "Commands (run from the repository root on one MI355X; OUT a scratch folder):", "",
             "```", cmd, "```", "",
             f"Calibration: the 1 GiB device copy in the same run reads FETCH_SIZE = {cf['FETCH_SIZE']:.0f} KiB and "
             f"WRITE_SIZE = {cw['WRITE_SIZE']:.0f} KiB, so FETCH_SIZE is scaled by {ff:.4f} and WRITE_SIZE by {fw:.4f}.",
             "", "Dispatches are grouped by kernel, grid size (blocks x threads) and bench phase (the "
             "decode batch is phase 1, after the plain streaming read of phase 0; each later workload packs its "
             "weights first and starts the next phase).", "",
             "| kernel | grid | phase | stage | calls | avg us | FETCH KiB/dispatch | WRITE KiB/dispatch | HBM bytes/dispatch (calibrated) |",
             "|---|---|---|---|---|---|---|---|---|"]
    rec = {"kernels_hip_sha256": hashlib.sha256(open(os.path.join(HERE, "csrc", "kernels.hip"), "rb").read()).hexdigest(),
           "fetch_scale": ff, "write_scale": fw, "kernels": {}}
    rows = sorted(kern.items(), key=lambda kv: -sum(kv[1]))
    # the stage's kernel of this workload: its (symbol, grid) of the longest mean duration (a bench run
    # that profiles prefill also times the decode batch first, whose launches are far shorter)
    best = {}
    for key, d in rows:
        st = stage_of(key[0])
        if st in STAGE.values() and (st not in best or sum(d) / len(d) > best[st][1]):
            best[st] = (key, sum(d) / len(d))
    for key, d in rows:
        n, g, ph = key
        st = stage_of(n)
        avg = sum(d) / len(d)
        fk = fetch.get(key, {}).get("FETCH_SIZE")
        wk = write.get(key, {}).get("WRITE_SIZE")
        tb = (fk * ff + wk * fw) * 1024 if fk is not None and wk is not None else None
        lines.append(f"| `{n[:78]}` | {g} | {ph} | {st or ''} | {len(d)} | {avg / 1000:.1f} | "
                     f"{'' if fk is None else f'{fk:.0f}'} | {'' if wk is None else f'{wk:.0f}'} | "
                     f"{'' if tb is None else f'{tb:.4g}'} |")
        if st in best and best[st][0] == key and tb is not None:
            rec["kernels"][st] = {"symbol": n, "grid": g, "phase": ph, "avg_us": avg / 1000, "fetch_kib": fk,
                                  "write_kib": wk, "hbm_bytes_per_launch": tb}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    open(os.path.join(ROOT, "profiles", f"kernels_{workload}.md"), "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w"), indent=1)
    print("\n".join(lines))

    # further counter passes: the stage kernels of this workload
    extra = sorted(glob.glob(os.path.join(run, "c*", "*_counter_collection.csv")))
    if not extra:
        return
    merged = collections.defaultdict(dict)
    for p in extra:
        per, _ = counter_passes(p)
        for k, c in per.items():
            merged[k].update(c)
    cl = [f"# On-chip counters: {workload}", "", "Commands (run from the repository root on one MI355X):", "", "```",
          cmd, "```", "",
          "Per dispatch, for the stage kernels of this workload (the same symbol and grid as in "
          f"`kernels_{workload}.md`). Normalisation: GRBM_GUI_ACTIVE summed over the 8 XCDs (its mean per XCD over "
          "the kernel's duration gives the clock); SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs; TA/TD/TCP "
          "busy and stall counts over the 256 CUs.", ""]
    for st, r in rec["kernels"].items():
        key = (r["symbol"], r["grid"], r["phase"])
        c = merged.get(key)
        if not c:
            continue
        cl += [f"## {st}: `{r['symbol']}` (grid {r['grid']}, {r['avg_us']:.1f} us)", "",
               "| derived | value |", "|---|---|"]
        for k, v in derived(c, r["avg_us"] * 1000).items():
            cl.append(f"| {k} | {v:.3f} |")
        cl += ["", "| counter | per dispatch |", "|---|---|"]
        for k in sorted(c):
            cl.append(f"| {k} | {c[k]:.4g} |")
        cl.append("")
    open(os.path.join(ROOT, "profiles", f"counters_{workload}.md"), "w").write("\n".join(cl) + "\n")
    print("\n".join(cl))


if __name__ == "__main__":
    main()

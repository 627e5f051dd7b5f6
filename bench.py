#!/usr/bin/env python3
"""Benchmark of the Kimi K3 LatentMoE layer forward on one MI355X.

Workload (default): K3-shape decode batch, T = 64 tokens, d = 7168, l = 3584, expert hidden 3072,
896 MXFP4 routed experts with top-16 sigmoid routing (b = 0), two full-width shared experts,
bf16 activations; seeded synthetic inputs (x ~ N(0, 1), weights ~ N(0, 1/fan_in) quantised to
MXFP4). A step is one full layer forward (x_gemm, topk, route, gateup, down, combine, y_gemm)
with inputs resident in HBM.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (the grouped gate/up GEMM:
HBM-bound at decode, MFMA-bound at prefill with MXFP8 activations) from per-stage HIP events
recorded on the launch stream over the timed region, the layer's HBM rate and MFMA fraction
(its time at the peaks of the dtypes each stage computes in, over the measured time), and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published (the scaled MFMA with an fp8 operand)
MXFP4_PEAK_TFLOPS = 10100.0    # MI355X dense MXFP4 (fp4 x fp4) scaled MFMA, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes recorded in
    profiles/, or None when the kernel source changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    src = os.path.join(ROOT, "latent_width_expert_amd", "csrc", "kernels.hip")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernels_hip_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes_per_launch"]


def load_summary(counts):
    """Per-expert token counts of one batch: the load histogram in brief."""
    import numpy as np
    c = np.sort(counts)[::-1]
    act = c[c > 0]
    return {"n_active": int(act.size), "mean": float(c.mean()), "max": int(c[0]),
            "p50_active": float(np.percentile(act, 50)) if act.size else 0.0,
            "p90_active": float(np.percentile(act, 90)) if act.size else 0.0,
            "top8": [int(v) for v in c[:8]],
            "hist_log2": {f"[{1 << b},{(1 << (b + 1)) - 1}]": int(((act >= (1 << b)) & (act < (1 << (b + 1)))).sum())
                          for b in range(int(np.log2(max(int(c[0]), 1))) + 1)}}


def mxfp4_bytes(n_elems: int) -> int:
    return n_elems // 2 + n_elems // 32


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3_decode_t64")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed region, run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs the layer on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    import workloads.device as wdev

    wl = workloads.get(args.workload)
    s = wl.shape
    T = wl.T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    moe = wdev.build_layer(wl, s, max_tokens=T, verbose=True)
    torch.cuda.synchronize()
    log(f"[bench] packed {moe.weight_bytes / 1e9:.2f} GB in {time.time() - t0:.1f} s")
    x = wdev.x_tensor(wl)
    y = torch.empty_like(x)

    for _ in range(args.warmup):
        moe.forward(x, y)
    torch.cuda.synchronize()

    # timed region: K steps on torch's current stream (the library launches on it), with the
    # library's per-stage events recorded on the same stream
    stream = torch.cuda.current_stream()
    moe.profile_begin(args.steps)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        moe.forward(x, y)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    stage_ms, calls = moe.profile_end()
    assert calls == args.steps
    ms_step = total_ms / args.steps
    stage_avg = {k: v / calls for k, v in stage_ms.items()}
    log(f"[bench] {ms_step:.4f} ms/step; stages (ms): " + ", ".join(f"{k} {v:.4f}" for k, v in stage_avg.items()))

    # routing of this batch (outside the timed region) for the algorithmic byte counts
    counts = torch.zeros(s.E, dtype=torch.int32, device=dev)
    moe.forward(x, y, taps={"counts": counts})
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    le = s.expert_in
    gu_bytes_expert = mxfp4_bytes(2 * s.h * le)
    dn_bytes_expert = mxfp4_bytes(le * s.h)
    dense_bytes = mxfp4_bytes(s.E * s.d) + s.Ns * mxfp4_bytes(3 * s.d * s.hs)
    if s.latent_moe:
        dense_bytes += 2 * mxfp4_bytes(s.d * s.l)
    rows = T * s.k
    act_b = 1 if s.act == "mxfp8" else 2
    # gate/up launch: weights of the active experts + dispatched z rows read + h written
    gu_alg = n_active * gu_bytes_expert + rows * le * act_b + rows * s.h * act_b
    layer_alg = n_active * (gu_bytes_expert + dn_bytes_expert) + dense_bytes + 2 * T * s.d * 2
    gu_ms = stage_avg["gateup"]
    flops_tok = 2 * (s.E * s.d + (2 * s.d * s.l if s.latent_moe else 0) + s.k * 3 * le * s.h + s.Ns * 3 * s.d * s.hs)
    # MFMA work per stage and the layer's time at the peaks of the dtypes the stages compute in
    dense_flops = 2 * T * (s.E * s.d + (2 * s.d * s.l if s.latent_moe else 0) + s.Ns * 3 * s.d * s.hs)
    routed_flops = 2 * rows * 3 * le * s.h
    routed_peak = FP8_PEAK_TFLOPS if s.act == "mxfp8" else BF16_PEAK_TFLOPS
    ideal_ms = (dense_flops / BF16_PEAK_TFLOPS + routed_flops / routed_peak) / 1e9
    gu_flops = 2 * rows * 2 * s.h * le
    traffic = recorded_traffic(wl.name, "gateup")
    if s.act == "mxfp8":
        # prefill: the grouped gate/up GEMM is MFMA-bound (MXFP8 x MXFP4 scaled MFMA at the fp8 rate)
        achieved = gu_flops / (gu_ms * 1e-3) / 1e12
        roofline = {"kernel": "gateup (grouped GLU gate/up GEMM, MXFP8 x MXFP4 scaled MFMA)", "bound": "mfma",
                    "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / FP8_PEAK_TFLOPS,
                    "traffic": traffic, "algorithmic_flops_per_launch": gu_flops,
                    "algorithmic_bytes_per_launch": gu_alg, "avg_launch_ms": gu_ms,
                    "frac_of_mxfp4_peak": achieved / MXFP4_PEAK_TFLOPS}
    else:
        achieved = gu_alg / (gu_ms * 1e-3) / 1e9
        roofline = {"kernel": "gateup (grouped GLU gate/up GEMM, MXFP4 weight stream)", "bound": "hbm",
                    "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": traffic, "algorithmic_bytes_per_launch": gu_alg, "avg_launch_ms": gu_ms}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_sample_tokens)

    out = {
        "metric": "LatentMoE layer tokens/s; decode HBM GB/s and prefill MFMA % of peak",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 x mxfp4" if s.act == "mxfp8" else "bf16 x mxfp4",
        "data": "synthetic (seeded: x ~ N(0,1) bf16; weights ~ N(0,1/fan_in) quantised to MXFP4)",
        "config": {"workload": wl.name, "tokens": T, "d": s.d, "latent": s.l if s.latent_moe else None,
                   "hidden": s.h, "experts": s.E, "top_k": s.k, "shared": s.Ns, "act": s.act,
                   "latent_moe": s.latent_moe, "weights": "MXFP4", "parallelism": "single GPU"},
        "roofline": roofline,
        "layer_hbm_gbps": layer_alg / (ms_step * 1e-3) / 1e9,
        "layer_hbm_frac": layer_alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_algorithmic_bytes": layer_alg,
        "layer_tflops": flops_tok * T / (ms_step * 1e-3) / 1e12,
        "layer_mfma_frac": ideal_ms / ms_step,
        "active_experts": n_active,
        "max_over_mean_load": float(counts.max() / max(counts.mean(), 1e-9)),
        "expert_load": load_summary(counts),
        "dispatch_values_per_token": s.k * le,
        "stages_ms": stage_avg,
        "cpu_baseline": cpu,
    }
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n
    print(json.dumps(out), flush=True)


class _CachedWeights:
    """The workload's tensors for the dense part and a given expert set, drawn before timing."""

    def __init__(self, wl, experts):
        self.wl = wl
        s = wl.shape
        self._dense = {"w_router": wl.w_router(), "bias": wl.router_bias()}
        if s.latent_moe:
            self._dense.update(w_down=wl.w_down(), w_up=wl.w_up(), gamma=wl.rms_gamma())
        self._shared = [wl.shared(j) for j in range(s.Ns)]
        self._experts = {int(e): wl.routed(int(e)) for e in experts}

    def w_router(self):
        return self._dense["w_router"]

    def w_down(self):
        return self._dense["w_down"]

    def w_up(self):
        return self._dense["w_up"]

    def router_bias(self):
        return self._dense["bias"]

    def rms_gamma(self):
        return self._dense["gamma"]

    def shared(self, j):
        return self._shared[j]

    def routed(self, e, count=1):
        return self._experts[int(e)]


def cpu_baseline(wl, n_tokens):
    """The fp64 oracle on the first n_tokens of the batch, on this host's cores."""
    import numpy as np

    from oracle import layer, mx

    s = wl.shape
    xb = wl.x_bits()[:n_tokens]
    # expert set of the sample (oracle router), drawn before timing
    Wr = layer.dequant(wl.w_router())
    sel = layer.select_topk(layer.router_scores(mx.bf16_from_bits(xb), Wr), wl.router_bias(), s.k)
    prov = _CachedWeights(wl, np.unique(sel.idx))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    t0 = time.perf_counter()
    layer.forward(xb, prov, s)
    dt = time.perf_counter() - t0
    log(f"[bench] oracle: {n_tokens} tokens in {dt:.1f} s")
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the {wl.name} batch (router over all 896 experts, "
                      f"{len(np.unique(sel.idx))} routed experts, all dense/shared matrices dequantised in fp64; "
                      f"numpy elementwise work single-threaded, BLAS on {threads} threads)",
            "seconds": dt}


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the Kimi K3 LatentMoE layer forward on one MI355X.

Headline workload (`value`): K3-shape decode batch, T = 64 tokens, d = 7168, l = 3584, expert hidden
3072, 896 MXFP4 routed experts with top-16 sigmoid routing (b = 0), two full-width shared experts,
bf16 activations; seeded synthetic inputs (x ~ N(0, 1), weights ~ N(0, 1/fan_in) quantised to MXFP4).
A step is one full layer forward (x_gemm, topk, route, gateup, down, combine, y_gemm) with inputs
resident in HBM.

The same run also measures, each on its own resident layer (one at a time):
  skewed      T = 512 with the Zipf router bias, literal (b = 1.5 ln w) and calibrated (b = 0.03 ln w)
  expert_parallel  one rank's share of an 8-way expert split (112 experts) on the rows it receives, at
              the decode and the prefill shapes
  lora        the decode batch with rank-16 BF16 LoRA deltas on every routed expert matrix
  prefill     T = 8192 with MXFP8 latent and hidden activations
  fullwidth   the conventional top-8 MoE at width 7168, T = 64 and T = 2048, with the LatentMoE layer at
              T = 2048 (bf16 activations) as its partner at the same dispatch payload
and the plain HBM read rate of a streaming kernel (k3moe_stream_read) as the practical ceiling.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (the grouped gate/up GEMM, HBM-
bound at decode and, by its arithmetic intensity, at prefill too) from per-stage HIP events recorded
on the launch stream over the timed region, the layer's HBM rate and MFMA fractions, the other
workloads' figures, and the CPU oracle timed on the whole decode batch with the GPU's parity
against it.
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
ALL = ("decode", "skewed", "ep", "lora", "prefill", "fullwidth")


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
            "max_over_mean": float(c[0] / max(c.mean(), 1e-9)),
            "p50_active": float(np.percentile(act, 50)) if act.size else 0.0,
            "p90_active": float(np.percentile(act, 90)) if act.size else 0.0,
            "top8": [int(v) for v in c[:8]],
            "hist_log2": {f"[{1 << b},{(1 << (b + 1)) - 1}]": int(((act >= (1 << b)) & (act < (1 << (b + 1)))).sum())
                          for b in range(int(np.log2(max(int(c[0]), 1))) + 1)}}


def mxfp4_bytes(n_elems: int) -> int:
    return n_elems // 2 + n_elems // 32


class Work:
    """Algorithmic work of one forward (counting rules: weights of the active experts and the dense
    matrices, x and y; the dispatched routed input read and the hidden written by the grouped GEMMs;
    FLOPs of useful MACs only)."""

    def __init__(self, s, T, counts):
        import numpy as np
        self.n_active = int((np.asarray(counts) > 0).sum())
        le = s.expert_in
        rows = T * s.k
        act_b = 1.03125 if s.act == "mxfp8" else 2.0
        self.gu_w = mxfp4_bytes(2 * s.h * le)
        self.dn_w = mxfp4_bytes(le * s.h)
        self.dense_w = mxfp4_bytes(s.E * s.d) + s.Ns * mxfp4_bytes(3 * s.d * s.hs)
        if s.latent_moe:
            self.dense_w += 2 * mxfp4_bytes(s.d * s.l)
        # gate/up launch: weights of the active experts + dispatched routed input read + hidden written
        self.gu_bytes = self.n_active * self.gu_w + rows * le * act_b + rows * s.h * act_b
        # down launch: weights + hidden read + expert outputs written (fp32)
        self.dn_bytes = self.n_active * self.dn_w + rows * s.h * act_b + rows * le * 4
        self.layer_bytes = self.n_active * (self.gu_w + self.dn_w) + self.dense_w + 2 * T * s.d * 2
        self.gu_flops = 2 * rows * 2 * s.h * le
        self.dn_flops = 2 * rows * s.h * le
        self.dense_flops = 2 * T * (s.E * s.d + (2 * s.d * s.l if s.latent_moe else 0) + s.Ns * 3 * s.d * s.hs)
        self.flops = self.dense_flops + self.gu_flops + self.dn_flops
        self.routed_peak = FP8_PEAK_TFLOPS if s.act == "mxfp8" else BF16_PEAK_TFLOPS


def roofline_of(kernel, bytes_, flops, ms, peak_tflops, traffic=None, stream_gbps=None):
    """Roofline of one launch: the bound is whichever of HBM bytes and MFMA work takes longer at the
    published peaks; achieved and frac are reported against that roof."""
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9) * 1e3
    t_mfma = flops / (peak_tflops * 1e12) * 1e3
    gbps = bytes_ / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    if t_hbm >= t_mfma:
        r = {"kernel": kernel, "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": gbps / HBM_PEAK_GBS}
    else:
        r = {"kernel": kernel, "bound": "mfma", "achieved": tflops, "peak": peak_tflops, "unit": "TFLOP/s",
             "frac": tflops / peak_tflops}
    r.update({"traffic": traffic, "algorithmic_bytes_per_launch": bytes_, "algorithmic_flops_per_launch": flops,
              "avg_launch_ms": ms, "roofline_ms": max(t_hbm, t_mfma), "gbps": gbps, "tflops": tflops,
              "frac_of_hbm_peak": gbps / HBM_PEAK_GBS, "frac_of_its_mfma_peak": tflops / peak_tflops})
    if stream_gbps:
        r["frac_of_stream_read"] = gbps / stream_gbps
    return r


def time_forward(moe, x, y, steps, warmup, profile=True):
    """Average ms per forward over `steps` timed calls (events on torch's current stream, the library
    launches on it), then -- with profile -- the library's per-stage averages over a second region of
    the same number of calls (its stage events add small gaps between launches, so the step time is
    taken without them). Returns (ms per step, stage averages, ms per step with the stage events)."""
    import torch
    for _ in range(warmup):
        moe.forward(x, y)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def region():
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(steps):
            moe.forward(x, y)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    ms = region()
    stages, ms_prof = None, None
    if profile:
        moe.profile_begin(steps)
        ms_prof = region()
        sm, calls = moe.profile_end()
        assert calls == steps
        stages = {k: v / calls for k, v in sm.items()}
    return ms, stages, ms_prof


def time_call(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def counts_of(moe, x, y, E):
    import torch
    c = torch.zeros(E, dtype=torch.int32, device=x.device)
    moe.forward(x, y, taps={"counts": c})
    torch.cuda.synchronize()
    return c.cpu().numpy()


def stream_read_gbps(dev):
    """Plain streaming read of 4 GiB (k3moe_stream_read): 2 warm-up calls, then 5 back to back."""
    import torch
    import latent_width_expert_amd as lwe
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    chk = torch.zeros(1, dtype=torch.int32, device=dev)
    ms = time_call(lambda: lwe.stream_read(buf, chk), 5, 2)
    del buf, chk
    return (4 << 30) / (ms * 1e-3) / 1e9


class CachingProvider:
    """A workload's weights, each routed chunk drawn once and kept on the host (the oracle's CPU run
    reuses the experts the GPU layer was packed from)."""

    chunked = True  # routed(e0, count) serves whole chunks (the device packer asks for them)

    def __init__(self, wl):
        self.wl = wl
        self.shape = wl.shape
        self.chunks = {}
        self.seed, self.T, self.name = wl.seed, wl.T, wl.name
        self._dense = {}

    def __getattr__(self, name):
        return getattr(self.wl, name)

    def routed(self, e0, count=1):
        for (c0, n), v in self.chunks.items():
            if c0 <= e0 and e0 + count <= c0 + n:
                return tuple((c[e0 - c0:e0 - c0 + count], s[e0 - c0:e0 - c0 + count]) for c, s in v)
        v = self.wl.routed(e0, count)
        self.chunks[(e0, count)] = v
        return v

    def w_router(self):
        if "r" not in self._dense:
            self._dense["r"] = self.wl.w_router()
        return self._dense["r"]

    def w_down(self):
        if "d" not in self._dense:
            self._dense["d"] = self.wl.w_down()
        return self._dense["d"]

    def w_up(self):
        if "u" not in self._dense:
            self._dense["u"] = self.wl.w_up()
        return self._dense["u"]

    def shared(self, j):
        if ("s", j) not in self._dense:
            self._dense[("s", j)] = self.wl.shared(j)
        return self._dense[("s", j)]


def gpu_gc():
    """Release device memory of layers the caller has dropped."""
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def decode_block(moe, wl, x, y, steps, warmup, stream_gbps):
    """Time one decode-like workload on a packed layer; its figures."""
    s = wl.shape
    T = x.shape[0]
    ms, stages, ms_prof = time_forward(moe, x, y, steps, warmup)
    counts = counts_of(moe, x, y, s.E)
    w = Work(s, T, counts)
    gu = stages["gateup"]
    rf = roofline_of("gateup (grouped GLU gate/up GEMM, MXFP4 weight stream)", w.gu_bytes, w.gu_flops, gu,
                     w.routed_peak, recorded_traffic(wl.name, "gateup"), stream_gbps)
    rf["step_ms_with_stage_events"] = ms_prof  # the region the stage durations come from
    return ms, stages, counts, w, rf


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default=",".join(ALL),
                    help="comma list of " + ",".join(ALL) + " (decode is always run: it is the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed regions, run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs the layer on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    configs = set(c.strip() for c in args.configs.split(",") if c.strip())
    bad = configs - set(ALL)
    if bad:
        print(json.dumps({"error": f"unknown configs {sorted(bad)}"}))
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    import workloads.device as wdev

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sec_steps = max(3, min(args.steps, 10))
    out = {}

    stream_gbps = stream_read_gbps(dev)
    log(f"[bench] plain streaming read: {stream_gbps:.0f} GB/s")

    # ---------------- decode (headline), skewed, expert-parallel rank, LoRA: the seed-1 weights
    wl = workloads.get("k3_decode_t64")
    s = wl.shape
    T = wl.T
    prov = CachingProvider(wl)
    t0 = time.time()
    moe = wdev.build_layer(prov, s, max_tokens=512, verbose=True)
    torch.cuda.synchronize()
    log(f"[bench] packed {moe.weight_bytes / 1e9:.2f} GB in {time.time() - t0:.1f} s")
    x = wdev.x_tensor(wl)
    y = torch.empty_like(x)
    ms_step, stage_avg, counts, w, roofline = decode_block(moe, wl, x, y, args.steps, args.warmup, stream_gbps)
    log(f"[bench] decode {ms_step:.4f} ms/step; stages (ms): " + ", ".join(f"{k} {v:.4f}" for k, v in stage_avg.items()))
    moe.forward(x, y)
    idx = torch.empty(T, s.k, dtype=torch.int32, device=dev)
    moe.forward(x, y, taps={"topk_idx": idx})
    torch.cuda.synchronize()
    y_dec = y.float().cpu().numpy().astype(np.float64)
    idx_dec = idx.cpu().numpy()

    if "skewed" in configs:
        sk = {}
        for name in ("k3_decode_t512_zipf", "k3_decode_t512_zipf_cal"):
            wz = workloads.get(name)
            moe.pack(dense=wdev.upload_dense(wz, wz.shape))
            torch.cuda.synchronize()
            xz = wdev.x_tensor(wz)
            yz = torch.empty_like(xz)
            ms, st, c, wk, rf = decode_block(moe, wz, xz, yz, sec_steps, 2, stream_gbps)
            sk[name] = {"tokens": wz.T, "zipf_alpha": wz.zipf_alpha, "ms_per_step": ms,
                        "tokens_per_s": wz.T / (ms * 1e-3), "layer_algorithmic_bytes": wk.layer_bytes,
                        "layer_hbm_gbps": wk.layer_bytes / (ms * 1e-3) / 1e9,
                        "layer_hbm_frac": wk.layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "gateup": rf, "stages_ms": st, "expert_load": load_summary(c)}
            log(f"[bench] {name}: {ms:.4f} ms/step, {sk[name]['layer_hbm_gbps']:.0f} GB/s, "
                f"max/mean {sk[name]['expert_load']['max_over_mean']:.2f}")
            if name == "k3_decode_t512_zipf":
                sk["quantile_balancing"] = quantile_balancing(moe, wz, xz, yz, c, sec_steps, stream_gbps)
        out["skewed"] = sk
        moe.pack(dense=wdev.upload_dense(wl, s))
        torch.cuda.synchronize()

    if "ep" in configs:
        out.setdefault("expert_parallel", {"ranks": 8, "experts_per_rank": s.E // 8})
        out["expert_parallel"]["decode"] = ep_rank(moe, prov, wl, x, sec_steps, stream_gbps)

    del moe
    gpu_gc()

    if "lora" in configs:
        wlo = workloads.get("k3_decode_t64_lora")
        lprov = CachingProvider(wlo)
        lprov.chunks = prov.chunks                     # same seed and shape: the same base experts
        lm = wdev.build_layer(lprov, wlo.shape, max_tokens=64, verbose=False)
        ms, st, c, wk, rf = decode_block(lm, wlo, x, y, sec_steps, 2, stream_gbps)
        r = wlo.shape.lora_rank
        lora_b = 2 * (2 * r * s.l + s.h * 2 * r + r * s.h + s.l * r)
        out["lora"] = {"workload": wlo.name, "rank": r, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
                       "extra_ms_vs_base": ms - ms_step, "lora_bytes_per_active_expert": lora_b,
                       "layer_algorithmic_bytes": wk.layer_bytes + wk.n_active * lora_b,
                       "layer_hbm_gbps": (wk.layer_bytes + wk.n_active * lora_b) / (ms * 1e-3) / 1e9,
                       "stages_ms": st}
        log(f"[bench] lora rank {r}: {ms:.4f} ms/step (+{ms - ms_step:.4f})")
        del lm, lprov
        gpu_gc()

    cpu, parity = (None, None)
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(prov, wl, y_dec, idx_dec)
    prov.chunks = {}
    del prov

    # ---------------- prefill (seed 3, MXFP8 activations)
    if "prefill" in configs:
        wp = workloads.get("k3_prefill_t8192")
        pp = CachingProvider(wp)
        pm = wdev.build_layer(pp, wp.shape, max_tokens=wp.T, verbose=False)
        xp = wdev.x_tensor(wp)
        yp = torch.empty_like(xp)
        ms, st, c, wk, _ = decode_block(pm, wp, xp, yp, sec_steps, 2, stream_gbps)
        gu = roofline_of("gateup (grouped GLU gate/up GEMM, MXFP8 x MXFP4 scaled MFMA)", wk.gu_bytes, wk.gu_flops,
                         st["gateup"], FP8_PEAK_TFLOPS, recorded_traffic(wp.name, "gateup"), stream_gbps)
        gu["frac_of_fp8_peak"] = gu["tflops"] / FP8_PEAK_TFLOPS
        gu["frac_of_mxfp4_peak"] = gu["tflops"] / MXFP4_PEAK_TFLOPS
        dn = roofline_of("down (grouped GLU down GEMM, MXFP8 x MXFP4 scaled MFMA)", wk.dn_bytes, wk.dn_flops,
                         st["down"], FP8_PEAK_TFLOPS, recorded_traffic(wp.name, "down"), stream_gbps)
        Tp = wp.T
        x_n = s.E + s.l + s.Ns * 2 * s.hs                 # outputs of the x-consumer GEMM (K = d)
        xg = roofline_of("x_gemm (router, W_down, shared gate/up; bf16 MFMA)",
                         mxfp4_bytes(x_n * s.d) + Tp * s.d * 2 + Tp * (4 * s.E + 1.03125 * s.l + 2 * s.Ns * s.hs),
                         2 * Tp * s.d * x_n, st["x_gemm"], BF16_PEAK_TFLOPS, recorded_traffic(wp.name, "x_gemm"),
                         stream_gbps)
        y_k = s.l + s.Ns * s.hs                           # reduction length of the output GEMM
        yg = roofline_of("y_gemm (W_up and shared downs; bf16 MFMA)", mxfp4_bytes(s.d * y_k) + Tp * y_k * 2 +
                         Tp * s.d * 2, 2 * Tp * s.d * y_k, st["y_gemm"], BF16_PEAK_TFLOPS,
                         recorded_traffic(wp.name, "y_gemm"), stream_gbps)
        roof_ms = gu["roofline_ms"] + dn["roofline_ms"] + xg["roofline_ms"] + yg["roofline_ms"] + \
            (Tp * s.k * s.l * 4 + Tp * s.l * 2) / (HBM_PEAK_GBS * 1e9) * 1e3
        layer_tf = wk.flops / (ms * 1e-3) / 1e12
        ideal_ms = (wk.dense_flops / BF16_PEAK_TFLOPS + (wk.gu_flops + wk.dn_flops) / FP8_PEAK_TFLOPS) / 1e9
        out["prefill"] = {"workload": wp.name, "tokens": Tp, "act": "mxfp8", "ms_per_step": ms,
                          "tokens_per_s": Tp / (ms * 1e-3), "roofline": gu, "down_roofline": dn,
                          "x_gemm_roofline": xg, "y_gemm_roofline": yg,
                          "layer_tflops": layer_tf, "layer_frac_of_mxfp4_peak": layer_tf / MXFP4_PEAK_TFLOPS,
                          "layer_mfma_frac": ideal_ms / ms, "layer_roofline_ms": roof_ms,
                          "layer_roofline_frac": roof_ms / ms, "stages_ms": st, "expert_load": load_summary(c)}
        log(f"[bench] prefill {ms:.3f} ms/step ({Tp / ms * 1e3:.0f} tok/s); gate/up {st['gateup']:.3f} ms = "
            f"{gu['frac']:.2f} of its {gu['bound']} roof; layer {layer_tf:.0f} TFLOP/s")
        if "ep" in configs:
            out.setdefault("expert_parallel", {"ranks": 8, "experts_per_rank": s.E // 8})
            out["expert_parallel"]["prefill"] = ep_rank(pm, pp, wp, xp, sec_steps, stream_gbps)
        del pm, pp, xp, yp
        gpu_gc()

    # ---------------- full width (seed 4): the conventional MoE at the same dispatch payload
    if "fullwidth" in configs:
        wf = workloads.get("fullwidth_t2048")
        fm = wdev.build_layer(wf, wf.shape, max_tokens=wf.T, verbose=False)
        fw = {}
        for Tf in (64, 2048):
            wft = wf.with_tokens(Tf)
            xf = wdev.x_tensor(wft)
            yf = torch.empty_like(xf)
            ms, st, c, wk, rf = decode_block(fm, wft, xf, yf, sec_steps, 2, stream_gbps)
            fw[f"t{Tf}"] = {"tokens": Tf, "top_k": wf.shape.k, "ms_per_step": ms, "tokens_per_s": Tf / (ms * 1e-3),
                            "layer_algorithmic_bytes": wk.layer_bytes,
                            "layer_hbm_gbps": wk.layer_bytes / (ms * 1e-3) / 1e9, "gateup": rf, "stages_ms": st,
                            "active_experts": wk.n_active,
                            "dispatch_values_per_token": wf.shape.k * wf.shape.expert_in}
            log(f"[bench] fullwidth T={Tf}: {ms:.3f} ms/step, {wk.layer_bytes / 1e9:.2f} GB")
        fw["vs_latent_t64"] = {"latent_ms": ms_step, "latent_bytes": w.layer_bytes,
                               "fullwidth_ms": fw["t64"]["ms_per_step"],
                               "fullwidth_bytes": fw["t64"]["layer_algorithmic_bytes"],
                               "speedup": fw["t64"]["ms_per_step"] / ms_step}
        del fm
        gpu_gc()
        # the LatentMoE partner at T = 2048 (K3 shape, bf16 activations, every expert active)
        wk3 = workloads.get("k3_t2048")
        km = wdev.build_layer(wk3, wk3.shape, max_tokens=wk3.T, verbose=False)
        xk = wdev.x_tensor(wk3)
        yk = torch.empty_like(xk)
        ms, st, c, wkk, rf = decode_block(km, wk3, xk, yk, sec_steps, 2, stream_gbps)
        fw["latent_t2048"] = {"workload": wk3.name, "tokens": wk3.T, "top_k": wk3.shape.k, "ms_per_step": ms,
                              "tokens_per_s": wk3.T / (ms * 1e-3), "layer_algorithmic_bytes": wkk.layer_bytes,
                              "layer_hbm_gbps": wkk.layer_bytes / (ms * 1e-3) / 1e9, "gateup": rf, "stages_ms": st,
                              "active_experts": wkk.n_active, "expert_load": load_summary(c),
                              "dispatch_values_per_token": wk3.shape.k * wk3.shape.expert_in}
        fw["vs_latent_t2048"] = {"latent_ms": ms, "latent_bytes": wkk.layer_bytes,
                                 "fullwidth_ms": fw["t2048"]["ms_per_step"],
                                 "fullwidth_bytes": fw["t2048"]["layer_algorithmic_bytes"],
                                 "speedup": fw["t2048"]["ms_per_step"] / ms}
        log(f"[bench] latent T=2048 (bf16): {ms:.3f} ms/step, {wkk.layer_bytes / 1e9:.2f} GB; full width "
            f"{fw['vs_latent_t2048']['speedup']:.2f}x slower")
        out["fullwidth"] = fw
        del km, xk, yk
        gpu_gc()

    res = {
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
        "dtype": "bf16 x mxfp4",
        "data": "synthetic (seeded: x ~ N(0,1) bf16; weights ~ N(0,1/fan_in) quantised to MXFP4)",
        "config": {"workload": wl.name, "tokens": T, "d": s.d, "latent": s.l, "hidden": s.h, "experts": s.E,
                   "top_k": s.k, "shared": s.Ns, "act": s.act, "latent_moe": s.latent_moe, "weights": "MXFP4",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stream_read_gbps": stream_gbps,
        "layer_hbm_gbps": w.layer_bytes / (ms_step * 1e-3) / 1e9,
        "layer_hbm_frac": w.layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_frac_of_stream_read": w.layer_bytes / (ms_step * 1e-3) / 1e9 / stream_gbps,
        "layer_algorithmic_bytes": w.layer_bytes,
        "layer_tflops": w.flops / (ms_step * 1e-3) / 1e12,
        "active_experts": w.n_active,
        "expert_load": load_summary(counts),
        "dispatch_values_per_token": s.k * s.expert_in,
        "stages_ms": stage_avg,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    res.update(out)
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = n
    print(json.dumps(res), flush=True)


def rank_loads(counts, n_ranks=8):
    """Rows each of n_ranks contiguous expert ranges receives: max over mean."""
    import numpy as np
    r = np.asarray(counts).reshape(n_ranks, -1).sum(axis=1)
    return float(r.max() / max(r.mean(), 1e-9))


def quantile_balancing(moe, wz, xz, yz, counts_before, steps, stream_gbps):
    """Quantile Balancing at K3 shape on the literal-Zipf router: the bias from the router scores of a
    held-out calibration batch (the next T tokens of the same stream) by k3moe_quantile_bias, packed
    in place of the Zipf bias, then the bench batch run with it. Each expert's calibration cutoff
    admits m = round(T k / E) tokens (s + b >= 0); the loads of the top-k selection are reported
    against the mean T k / E, per expert and per contiguous range of E / 8 experts."""
    import numpy as np
    import torch
    import workloads.device as wdev
    s = wz.shape
    cal = torch.from_numpy(wz.x_bits(2 * wz.T)[wz.T:].view(np.int16)).to(xz.device).view(torch.bfloat16)
    scores = torch.empty(wz.T, s.E, dtype=torch.float32, device=xz.device)
    moe.forward(cal, torch.empty_like(cal), taps={"scores": scores})
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    bias = moe.quantile_bias(scores)
    ev1.record()
    torch.cuda.synchronize()
    cal_ms = ev0.elapsed_time(ev1)
    # cutoff check on the calibration batch: tokens with s + b >= 0 per expert
    admitted = ((scores + bias[None, :]) >= 0).sum(dim=0).cpu().numpy()
    dense = wdev.upload_dense(wz, s)
    dense["router_bias"] = bias
    moe.pack(dense=dense)
    torch.cuda.synchronize()
    ms, st, c, wk, rf = decode_block(moe, wz, xz, yz, steps, 2, stream_gbps)
    moe.pack(dense=wdev.upload_dense(wz, s))
    torch.cuda.synchronize()
    target = wz.T * s.k / s.E
    q = {"calibration_tokens": wz.T, "m": int(np.floor(target + 0.5)), "count_target_Tk_over_E": target,
         "calibration_ms": cal_ms,
         "admitted_per_expert_min_max": [int(admitted.min()), int(admitted.max())],
         "before": {"expert_load": load_summary(counts_before), "rank_max_over_mean": rank_loads(counts_before)},
         "after": {"expert_load": load_summary(c), "rank_max_over_mean": rank_loads(c), "ms_per_step": ms,
                   "layer_hbm_gbps": wk.layer_bytes / (ms * 1e-3) / 1e9, "stages_ms": st},
         "experts_within_2x_of_target": float(((c >= target / 2) & (c <= 2 * target)).mean())}
    log(f"[bench] quantile balancing (T={wz.T}, m={q['m']}): expert max/mean "
        f"{q['before']['expert_load']['max_over_mean']:.2f} -> {q['after']['expert_load']['max_over_mean']:.2f}, "
        f"active {q['before']['expert_load']['n_active']} -> {q['after']['expert_load']['n_active']}, "
        f"rank max/mean {q['before']['rank_max_over_mean']:.2f} -> {q['after']['rank_max_over_mean']:.2f}, "
        f"{ms:.4f} ms/step")
    return q


def ep_rank(moe, prov, wl, x, steps, stream_gbps, n_ranks=8, rank=0):
    """One rank of an n_ranks expert split: its experts packed alone, timed on the rows the head sends
    it (k3moe_experts_forward)."""
    import torch
    import workloads.device as wdev
    s = wl.shape
    per = s.E // n_ranks
    rows, scales, send, counts = moe.forward_head(x, n_ranks)
    torch.cuda.synchronize()
    send = send.cpu().numpy()
    start, R = int(send[:rank].sum()), int(send[rank])
    lc = counts[rank * per:(rank + 1) * per].contiguous()
    loc = wdev.build_layer(prov, s, max_tokens=x.shape[0], experts=range(rank * per, (rank + 1) * per), dense=False)
    r_rows = rows[start:start + R].contiguous()
    r_sc = scales[start:start + R].contiguous() if scales is not None else None
    o = torch.empty(R, s.expert_in, dtype=torch.float32, device=x.device)
    ms = time_call(lambda: loc.experts_forward(r_rows, r_sc, lc, out=o), steps, 2)
    c = lc.cpu().numpy()
    n_act = int((c > 0).sum())
    act_b = 1.03125 if s.act == "mxfp8" else 2.0
    wb = n_act * mxfp4_bytes(3 * s.h * s.expert_in) + R * s.expert_in * act_b + R * s.expert_in * 4
    fl = 2 * R * 3 * s.h * s.expert_in
    peak = FP8_PEAK_TFLOPS if s.act == "mxfp8" else BF16_PEAK_TFLOPS
    r = roofline_of(f"experts of rank {rank} of {n_ranks} (gate/up + down)", wb, fl, ms, peak, None, stream_gbps)
    log(f"[bench] {wl.name} rank {rank}/{n_ranks}: {R} rows on {per} experts ({n_act} active) in {ms:.3f} ms "
        f"({r['frac']:.2f} of its {r['bound']} roof)")
    res = {"workload": wl.name, "rank": rank, "rows": R, "rows_per_token_share": R / x.shape[0],
           "send_counts": send.tolist(), "active_local_experts": n_act, "ms": ms, "roofline": r}
    del loc, rows, scales, r_rows, r_sc, o
    gpu_gc()
    return res


def cpu_baseline(prov, wl, y_gpu, idx_gpu):
    """The fp64 oracle on the whole decode batch on this host's cores, and the GPU's parity against it
    (the output bar: relative L2 <= 5e-3, max-abs <= 2e-2 rms(y); tokens whose GPU selection differs
    inside the key-tie tolerance scored against the oracle run with the GPU's selection)."""
    import numpy as np

    from oracle import layer

    s = wl.shape
    xb = wl.x_bits()
    T = xb.shape[0]
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    # every routed expert already drawn (the packing drew them): the timed region is the oracle alone
    t0 = time.perf_counter()
    ref = layer.forward(xb, prov, s, keep_expert_rows=False)
    dt = time.perf_counter() - t0
    log(f"[bench] oracle: {T} tokens in {dt:.1f} s")
    ok, flip = layer.check_selection(idx_gpu, ref.taps["selection"], tol=1e-6)
    yref = ref.y
    if flip.any():
        r2 = layer.forward(xb[flip], prov, s, select_override={i: idx_gpu[t] for i, t in enumerate(np.nonzero(flip)[0])},
                           keep_expert_rows=False)
        yref = yref.copy()
        yref[flip] = r2.y
    rel = float(np.linalg.norm(y_gpu - yref) / np.linalg.norm(yref))
    ma = float(np.max(np.abs(y_gpu - yref)) / np.sqrt(np.mean(yref ** 2)))
    cpu = {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole {T}-token {wl.name} batch (router over all {s.E} experts, "
                     f"{int((ref.taps['counts'] > 0).sum())} routed experts dequantised one at a time, every dense "
                     f"and shared matrix, fp64; numpy elementwise work single-threaded, BLAS on {threads} threads)",
           "seconds": dt}
    parity = {"tokens": T, "y_rel_l2": rel, "y_maxabs_over_rms": ma, "selection_ok": bool(ok.all()),
              "flipped_tokens": int(flip.sum()), "bar": {"rel_l2": 5e-3, "maxabs_over_rms": 2e-2},
              "pass": bool(ok.all() and rel <= 5e-3 and ma <= 2e-2)}
    log(f"[bench] parity over {T} tokens: y rel L2 {rel:.2e}, max-abs/rms {ma:.2e}")
    return cpu, parity


if __name__ == "__main__":
    main()

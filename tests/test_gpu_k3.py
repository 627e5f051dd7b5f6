"""GPU parity at K3 shape (d = 7168, l = 3584, hidden 3072, E = 896, k = 16, two shared experts), in
the launch configuration the benchmark times.

Every token: router scores, selection (exact up to oracle key ties < 1e-6, counted), p, counts,
offsets, permutation and inverse (bit-exact), and the latent z at its quantisation point (bf16
or MXFP8 codes: strict against the oracle's encoder on the GPU's fp32 values, end to end
against the oracle's own values, boundary codes counted).
Outputs: the decode batch of 64 tokens whole (y, u, n and the shared hidden of every token against
the oracle's forward); the skewed, full-width and T = 2048 batches on 16 tokens spread through the
batch, the skewed and T = 2048 ones also stage-wise on every row of experts from each kernel band; the
prefill chunk stage-wise on every dispatched row of 64 experts spread over the id range (the
hottest, ids above 512, a count that is not a multiple of the 192-row chunk) and end to end on 64
tokens spread through the batch. Also the BF16 LoRA variant at decode and the expert-parallel split
(one rank's 112 experts on its rows) at decode and prefill. One packed layer is resident at a time.
"""
from __future__ import annotations

import gc
import sys

import numpy as np
import pytest
import torch

import workloads
import workloads.device as wdev
from oracle import layer, mx
from tests import parity

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.__stderr__, flush=True)


_CUR = {"key": None, "moe": None}


def get_layer(wl, max_tokens):
    """Packed layer for the workload's seed, shape and activation format (bias re-packed)."""
    key = (wl.seed, wl.shape, max_tokens)
    if _CUR["key"] != key:
        _CUR["moe"] = None
        _CUR.pop("rank", None)
        gc.collect()
        torch.cuda.empty_cache()
        _log(f"[k3] packing seed {wl.seed} {wl.shape}")
        _CUR["moe"] = wdev.build_layer(wl, wl.shape, max_tokens=max_tokens, verbose=True)
        _CUR["key"] = key
        _CUR["bias"] = wl.bias, wl.zipf_alpha
    if _CUR.get("bias") != (wl.bias, wl.zipf_alpha):
        _CUR["moe"].pack(dense=wdev.upload_dense(wl, wl.shape))
        torch.cuda.synchronize()
        _CUR["bias"] = wl.bias, wl.zipf_alpha
    return _CUR["moe"]


def run_taps(moe, wl, T, rows=False):
    s = wl.shape
    f8 = s.act == "mxfp8"
    dev = "cuda"
    t = dict(scores=torch.empty(T, s.E, dtype=torch.float32, device=dev),
             topk_idx=torch.empty(T, s.k, dtype=torch.int32, device=dev),
             topk_p=torch.empty(T, s.k, dtype=torch.float32, device=dev),
             counts=torch.empty(s.E, dtype=torch.int32, device=dev),
             offsets=torch.empty(s.E + 1, dtype=torch.int32, device=dev),
             perm=torch.empty(T * s.k, dtype=torch.int32, device=dev),
             inv=torch.empty(T * s.k, dtype=torch.int32, device=dev),
             u=torch.empty(T, s.expert_in, dtype=torch.float32, device=dev))
    if s.latent_moe:
        t.update(z=torch.empty(T, s.l, dtype=torch.uint8 if f8 else torch.bfloat16, device=dev),
                 z_f32=torch.empty(T, s.l, dtype=torch.float32, device=dev),
                 n=torch.empty(T, s.l, dtype=torch.bfloat16, device=dev))
        if f8:
            t["z_scales"] = torch.empty(T, s.l // 32, dtype=torch.uint8, device=dev)
    if s.Ns:
        t["hs"] = torch.empty(T, s.Ns * s.hs, dtype=torch.bfloat16, device=dev)
    if rows:
        t.update(h=torch.empty(T * s.k, s.h, dtype=torch.uint8 if f8 else torch.bfloat16, device=dev),
                 h_f32=torch.empty(T * s.k, s.h, dtype=torch.float32, device=dev),
                 expert_out=torch.empty(T * s.k, s.expert_in, dtype=torch.float32, device=dev))
        if f8:
            t["h_scales"] = torch.empty(T * s.k, s.h // 32, dtype=torch.uint8, device=dev)
    x = wdev.x_tensor(wl, T)
    y = moe.forward(x, taps=t)
    torch.cuda.synchronize()
    g = {k: (parity.bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in t.items()}
    del t
    g["y"] = parity.np64(y)
    return g


def spread(T, n, extra=()):
    """n token indices spread evenly through [0, T), plus some chosen ones."""
    return sorted(set(np.linspace(0, T - 1, n).round().astype(int).tolist()) | set(extra))


def check_layer(wl, sample, max_tokens=None, rows=False):
    s = wl.shape
    T = wl.T
    moe = get_layer(wl, max_tokens or T)
    _log(f"[k3] {wl.name}: GPU forward T={T}")
    g = run_taps(moe, wl, T, rows=rows)
    xb = wl.x_bits()
    xh = mx.bf16_from_bits(xb)
    # router over every token
    sc = layer.router_scores(xh, layer.dequant(wl.w_router()))
    assert np.max(np.abs(g["scores"] - sc)) < 1e-5
    sel = layer.select_topk(sc, wl.router_bias(), s.k)
    flips = parity.check_routing(g, sel, s.E)
    gidx = g["topk_idx"].astype(np.int64)
    assert np.max(np.abs(g["topk_p"] - layer.renorm(sc, gidx))) < 1e-5
    counts = g["counts"]
    _log(f"[k3] {wl.name}: routing ok, flips {flips}, active experts {(counts > 0).sum()}, "
         f"max/mean load {counts.max() / counts.mean():.2f}")
    # latent z of every token at its quantisation point; tokens with a boundary code marked
    zdirty = np.zeros(T, bool)
    if s.latent_moe:
        Wd = layer.dequant(wl.w_down())
        aWd = np.abs(Wd)
        nz = 0
        for r0 in range(0, T, 1024):
            xs = xh[r0:r0 + 1024]
            z = xs @ Wd.T
            bound = parity.dot_error_bound(np.abs(xs), aWd)
            sl = slice(r0, r0 + 1024)
            if s.act == "mxfp8":
                nz += parity.check_mx_quant(g["z"][sl], g["z_scales"][sl], g["z_f32"][sl], z, bound)
                c3, s3 = mx.mx_quantize(z, "e4m3")
                zdirty[sl] = (c3 != g["z"][sl]).any(axis=1) | (s3 != g["z_scales"][sl]).any(axis=1)
            else:
                nz += parity.check_bf16_quant(g["z"][sl], g["z_f32"][sl], z, bound)
                zdirty[sl] = (mx.bf16_round(z) != mx.bf16_from_bits(g["z"][sl])).any(axis=1)
        assert nz <= 1e-3 * T * s.l + 2
        _log(f"[k3] {wl.name}: z quantisation ok ({nz} boundary codes in {int(zdirty.sum())} tokens)")
    # sampled tokens through the whole layer: against the oracle's own chain (full bar; selection of
    # flipped tokens taken from the GPU), and for MXFP8 also against the oracle taking the GPU's codes
    ov = {i: gidx[t] for i, t in enumerate(sample)}
    _log(f"[k3] {wl.name}: oracle forward on {len(sample)} tokens")
    ref = layer.forward(xb[sample], wl, s, select_override=ov, keep_expert_rows=False)
    clean = np.array([not zdirty[t] for t in sample])
    if s.act == "mxfp8":
        # tokens whose z codes all equal the oracle's: the full bar against the oracle's own chain; the
        # others (a code across a rounding boundary inside the fp32 bound): the full bar against the
        # oracle taking the GPU's z and h codes
        assert clean.sum() >= min(8, len(sample)), f"{clean.sum()} clean tokens"
        rel, ma = parity.assert_y(g["y"][sample][clean], ref.y[clean], "y (clean tokens)")
        dirty = [t for t in sample if zdirty[t]]
        if rows and dirty:
            rsel = g["inv"].reshape(T, s.k)[dirty]                      # [n, k] dispatched rows
            hq = parity.decode_act(g["h"][rsel.reshape(-1)], g["h_scales"][rsel.reshape(-1)], "mxfp8")
            zq = parity.decode_act(g["z"][dirty], g["z_scales"][dirty], "mxfp8")
            ovd = {i: gidx[t] for i, t in enumerate(dirty)}
            refq = layer.forward(xb[dirty], wl, s, select_override=ovd, keep_expert_rows=False, z_override=zq,
                                 h_override=hq.reshape(len(dirty), s.k, s.h))
            rq, mq = parity.assert_y(g["y"][dirty], refq.y, "y (oracle on the GPU's codes)")
            _log(f"[k3] {wl.name}: {len(dirty)} tokens with a boundary z code vs oracle on the GPU's codes: "
                 f"rel L2 {rq:.2e}, max-abs/rms {mq:.2e}")
    else:
        rel, ma = parity.assert_y(g["y"][sample], ref.y, "y")
    parity.assert_y(g["u"][sample][clean], ref.taps["u"][clean], "u")
    if s.latent_moe:
        parity.assert_y(mx.bf16_from_bits(g["n"][sample][clean]), ref.taps["n"][clean], "n")
    if s.Ns:
        parity.assert_y(mx.bf16_from_bits(g["hs"][sample]), np.concatenate(ref.taps["hs"], axis=1), "shared")
    _log(f"[k3] {wl.name}: {len(sample)} sampled tokens ({int(clean.sum())} without a boundary code): "
         f"y rel L2 {rel:.2e}, max-abs/rms {ma:.2e}")
    return g


def stagewise_experts(wl, g, experts):
    """Every dispatched row of the given experts: the gate/up + SwiGLU values against the oracle's step
    on the GPU's own quantised latent (element-wise within the fp32 bound), and the down projection
    against the oracle on the GPU's own quantised hidden (relative L2 <= 1e-4, R26)."""
    s = wl.shape
    perm, offsets = g["perm"].astype(np.int64), g["offsets"]
    zq = parity.decode_act(g["z"], g.get("z_scales"), s.act)
    worst_h, worst_o, rows = 0.0, 0.0, 0
    for e in experts:
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        G, U, D = (layer.dequant(m) for m in parity._first3(wl.routed(int(e))))
        h_ex, hb = parity.glu_hidden_bound(zq[perm[r0:r1]], G, U, layer.lora_factors(wl, int(e), s),
                                           scaled_mfma=s.act == "mxfp8")
        err = np.abs(g["h_f32"][r0:r1] - h_ex)
        worst_h = max(worst_h, float(np.max(err / hb)))
        assert np.all(err <= hb), f"expert {e}: hidden off by {np.max(err / hb):.3g} x the bound"
        hq = parity.decode_act(g["h"][r0:r1], g["h_scales"][r0:r1] if "h_scales" in g else None, s.act)
        o_ref = hq @ D.T
        rel = parity.rel_l2(g["expert_out"][r0:r1], o_ref)
        worst_o = max(worst_o, rel)
        assert rel < 1e-4, (e, rel)
        rows += r1 - r0
    return worst_h, worst_o, rows


@pytest.mark.timeout(900)
def test_k3_decode_t64_every_token():
    """The decode batch whole: every token's y, u, n and shared hidden against the oracle."""
    wl = workloads.get("k3_decode_t64")
    check_layer(wl, list(range(64)), max_tokens=512)


@pytest.mark.timeout(900)
def test_k3_expert_parallel_rank_decode():
    _rank_check(workloads.get("k3_decode_t64"), rank=3)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["k3_decode_t512_zipf", "k3_decode_t512_zipf_cal"])
def test_k3_decode_t512_skewed(name):
    """16 spread tokens end to end; stage-wise, every row of experts from each kernel band: below 16 rows
    (panel kernel, shared A tile), 16-63 (mid-row kernel), 64 and more (row-tiled kernel)."""
    wl = workloads.get(name)
    g = check_layer(wl, spread(512, 16, extra=(5,)), max_tokens=512, rows=True)
    c = g["counts"]
    assert c.sum() == 512 * 16
    experts = band_experts(c, 4)
    wh, wo, rows = stagewise_experts(wl, g, experts)
    _log(f"[k3] {name} stage-wise: experts {experts} (rows {[int(c[e]) for e in experts]}): hidden within "
         f"{wh:.3f} x its bound, expert outputs rel L2 <= {wo:.2e}")


def band_experts(c, n):
    """Up to n experts from each row band of the grouped kernels (1-15, 16-63, 64 and more rows), the
    smallest and largest of each band first."""
    out = []
    for lo, hi in ((1, 16), (16, 64), (64, 1 << 30)):
        ids = [int(e) for e in np.argsort(c, kind="stable") if lo <= c[e] < hi]
        if ids:
            mid = ids[1:-1]
            pick = [ids[0], ids[-1]] + mid[:: max(1, len(mid) // max(1, n - 2))][: max(0, n - 2)]
            out += pick
    return sorted(set(out))


@pytest.mark.timeout(900)
def test_k3_prefill_t8192_mxfp8():
    """Prefill chunk: every row of 64 experts spread over the id range stage-wise; 64 spread tokens
    end to end."""
    wl = workloads.get("k3_prefill_t8192")
    g = check_layer(wl, spread(8192, 64), rows=True)
    c = g["counts"]
    hot = int(np.argmax(c))
    ragged = [int(e) for e in np.nonzero(c % 192 != 0)[0] if e >= 512][:4]
    experts = sorted(set(np.linspace(0, 895, 64).round().astype(int).tolist()) | {hot} | set(ragged) |
                     set(range(512, 516)))
    assert len(experts) >= 64
    wh, wo, rows = stagewise_experts(wl, g, experts)
    _log(f"[k3] prefill stage-wise: {len(experts)} experts (hottest {hot} with {c[hot]} rows), {rows} rows: "
         f"hidden within {wh:.3f} x its bound, expert outputs rel L2 <= {wo:.2e}")


@pytest.mark.timeout(900)
def test_k3_expert_parallel_rank_prefill():
    _rank_check(workloads.get("k3_prefill_t8192"), rank=5)


@pytest.mark.timeout(900)
def test_k3_decode_repeat_bit_identical():
    """Determinism at K3 shape: two forwards give identical y and permutation."""
    wl = workloads.get("k3_prefill_t8192").with_tokens(1024)
    moe = get_layer(workloads.get("k3_prefill_t8192"), 8192)
    x = wdev.x_tensor(wl)
    perm = [torch.empty(1024 * 16, dtype=torch.int32, device="cuda") for _ in range(2)]
    y1 = moe.forward(x, taps={"perm": perm[0]})
    y2 = moe.forward(x, taps={"perm": perm[1]})
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(perm[0], perm[1])


def _rank_check(wl, rank, n_ranks=8):
    """One expert-parallel rank: its 112 experts on a context of their own, run on the rows the head
    sends it, reproduce the full layer's expert outputs for those rows bit for bit (same kernels on the
    same rows), and the send side matches the oracle (counts exactly, rows bit for bit)."""
    s = wl.shape
    T = wl.T
    full = get_layer(wl, T if T > 64 else 512)
    per = s.E // n_ranks
    key = ("rank", wl.seed, s, rank)
    if _CUR.get("rank", (None,))[0] != key:
        _CUR.pop("rank", None)
        gc.collect()
        _log(f"[k3] packing rank {rank} of {n_ranks}: experts {rank * per}..{(rank + 1) * per - 1}")
        _CUR["rank"] = (key, wdev.build_layer(wl, s, max_tokens=T, experts=range(rank * per, (rank + 1) * per),
                                              dense=False))
    loc = _CUR["rank"][1]
    x = wdev.x_tensor(wl)
    taps = {"expert_out": torch.empty(T * s.k, s.l, dtype=torch.float32, device="cuda"),
            "perm": torch.empty(T * s.k, dtype=torch.int32, device="cuda"),
            "topk_idx": torch.empty(T, s.k, dtype=torch.int32, device="cuda")}
    if s.act == "mxfp8":
        taps.update(z=torch.empty(T, s.l, dtype=torch.uint8, device="cuda"),
                    z_scales=torch.empty(T, s.l // 32, dtype=torch.uint8, device="cuda"))
    else:
        taps["z"] = torch.empty(T, s.l, dtype=torch.bfloat16, device="cuda")
    full.forward(x, taps=taps)
    rows, scales, send, counts = full.forward_head(x, n_ranks)
    torch.cuda.synchronize()
    idx = taps["topk_idx"].cpu().numpy()
    send_np = send.cpu().numpy()
    assert send_np.tolist() == layer.ep_send_counts(idx, s.E, n_ranks).tolist()
    perm = taps["perm"].cpu().long()
    if s.act == "mxfp8":
        assert torch.equal(rows.cpu(), taps["z"].cpu()[perm]) and torch.equal(scales.cpu(), taps["z_scales"].cpu()[perm])
    else:
        assert torch.equal(rows.view(torch.int16).cpu(), taps["z"].view(torch.int16).cpu()[perm])
    start = int(send_np[:rank].sum())
    R = int(send_np[rank])
    sl = slice(start, start + R)
    out = loc.experts_forward(rows[sl], scales[sl] if scales is not None else None,
                              counts[rank * per:(rank + 1) * per].contiguous())
    torch.cuda.synchronize()
    same = torch.equal(out.view(torch.int32).cpu(), taps["expert_out"][sl].view(torch.int32).cpu())
    assert same, "rank outputs differ from the full layer's"
    _log(f"[k3] {wl.name}: rank {rank}/{n_ranks}: {R} rows over {per} experts "
         f"({int((counts[rank * per:(rank + 1) * per] > 0).sum())} active): bit-identical to the full layer")


@pytest.mark.timeout(900)
def test_k3_t2048_bf16():
    """K3 shape, 2048 tokens, bf16 activations (20-56 rows per expert: the mid-row kernel, the larger
    experts on the row-tiled kernel): 16 spread tokens end to end, every row of experts from each band
    stage-wise."""
    wl = workloads.get("k3_t2048")
    g = check_layer(wl, spread(2048, 16), rows=True)
    c = g["counts"]
    experts = band_experts(c, 6)
    wh, wo, rows = stagewise_experts(wl, g, experts)
    _log(f"[k3] k3_t2048 stage-wise: experts {experts} (rows {[int(c[e]) for e in experts]}): hidden within "
         f"{wh:.3f} x its bound, expert outputs rel L2 <= {wo:.2e}")


@pytest.mark.timeout(900)
def test_k3_decode_t64_lora():
    """Rank-16 BF16 LoRA deltas on every routed expert matrix, decode batch: 16 spread tokens."""
    check_layer(workloads.get("k3_decode_t64_lora"), spread(64, 16))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [64, 2048])
def test_fullwidth(T):
    wl = workloads.get("fullwidth_t2048").with_tokens(T)
    check_layer(wl, spread(T, 16), max_tokens=2048)

"""GPU parity on the small layers: every intermediate of the HIP path against the fp64 oracle.

Sizes: tiny LatentMoE (T = 64, d = 256, l = 128, hidden 96, E = 16, k = 4, one shared expert)
and variants (MXFP8 activations, full-width conventional MoE, skewed bias with two shared
experts, MXFP8 or bf16 with many rows per expert over several K windows and row chunks, a skewed
load split between the row-tiled and the panel kernels); ragged token counts cover partial 16-row
tiles and partial row chunks.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import layer, mx
from tests import parity
from tests.weightset import ArrayWeights

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _taps(shape, T, device="cuda"):
    s = shape
    le = s.expert_in
    Tk = T * s.k
    f8 = s.act == "mxfp8"
    z = lambda *sh, dt: torch.zeros(*sh, dtype=dt, device=device)  # noqa: E731
    t = dict(scores=z(T, s.E, dt=torch.float32), topk_idx=z(T, s.k, dt=torch.int32),
             topk_p=z(T, s.k, dt=torch.float32), counts=z(s.E, dt=torch.int32), offsets=z(s.E + 1, dt=torch.int32),
             perm=z(Tk, dt=torch.int32), inv=z(Tk, dt=torch.int32),
             h=z(Tk, s.h, dt=torch.uint8 if f8 else torch.bfloat16), h_f32=z(Tk, s.h, dt=torch.float32),
             expert_out=z(Tk, le, dt=torch.float32), u=z(T, le, dt=torch.float32))
    if f8:
        t["h_scales"] = z(Tk, s.h // 32, dt=torch.uint8)
    if s.latent_moe:
        t.update(z=z(T, s.l, dt=torch.uint8 if f8 else torch.bfloat16), z_f32=z(T, s.l, dt=torch.float32),
                 n=z(T, s.l, dt=torch.bfloat16))
        if f8:
            t["z_scales"] = z(T, s.l // 32, dt=torch.uint8)
    if s.Ns:
        t["hs"] = z(T, s.Ns * s.hs, dt=torch.bfloat16)
    return t


def run_gpu(moe, wl, T):
    x = workloads.device.x_tensor(wl, T)
    taps = _taps(wl.shape, T)
    y = moe.forward(x, taps=taps)
    torch.cuda.synchronize()
    out = {k: (parity.bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in taps.items()}
    out["y"] = parity.np64(y)
    return out


_CASES = {}


def case(name):
    if name not in _CASES:
        import workloads.device  # noqa: F401
        wl = workloads.get(name)
        w = ArrayWeights(wl)
        _log(f"[case] {name}: packing")
        moe = workloads.device.build_layer(w, wl.shape, max_tokens=wl.T)
        _CASES[name] = (wl, w, moe)
    return _CASES[name]


def check_all(name, T):
    wl, w, moe = case(name)
    s = wl.shape
    _log(f"[check] {name} T={T}")
    g = run_gpu(moe, wl, T)
    ref = layer.forward(wl.x_bits(T), w, s)
    rt = ref.taps
    # router: fp32 scores vs fp64
    assert np.max(np.abs(g["scores"] - rt["scores"])) < 2e-6
    flips = parity.check_routing(g, rt["selection"], s.E)
    gidx = g["topk_idx"].astype(np.int64)
    p_ref = layer.renorm(rt["scores"], gidx)
    assert np.max(np.abs(g["topk_p"] - p_ref)) < 2e-6
    if flips:
        ref = layer.forward(wl.x_bits(T), w, s, select_override={t: gidx[t] for t in range(T)})
        rt = ref.taps
    f8 = s.act == "mxfp8"
    perm = g["perm"].astype(np.int64)
    # latent z at its quantisation point: strict encoding of the GPU's own values, the values within
    # the fp32 accumulation bound of the oracle's, and the tokens whose codes differ from the oracle's
    # own encoding (a rounding boundary inside that bound) marked
    zdirty = np.zeros(T, bool)
    if s.latent_moe:
        xh = mx.bf16_from_bits(wl.x_bits(T))
        bound = parity.dot_error_bound(np.abs(xh), np.abs(layer.dequant(w.w_down())))
        if f8:
            nz = parity.check_mx_quant(g["z"], g["z_scales"], g["z_f32"], rt["z"], bound)
            zdirty = (parity.decode_act(g["z"], g["z_scales"], "mxfp8") != rt["zq"]).any(axis=1)
        else:
            nz = parity.check_bf16_quant(g["z"], g["z_f32"], rt["z"], bound)
            zdirty = (mx.bf16_from_bits(g["z"]) != rt["zq"]).any(axis=1)
        assert nz <= max(2, 1e-3 * g["z_f32"].size)
    # GLU hidden (dispatched row order): strict quantisation of the GPU's own values; on the rows of
    # tokens whose z equals the oracle's, the GPU's values within the fp32 bound of the oracle's and
    # the codes that differ from the oracle's own encoding counted (boundary cases inside the bound)
    if f8:
        c2, s2 = mx.mx_quantize(g["h_f32"].astype(np.float64), "e4m3")
        assert np.array_equal(c2, g["h"]) and np.array_equal(s2, g["h_scales"])
    else:
        assert np.array_equal(mx.bf16_round(g["h_f32"].astype(np.float64)), mx.bf16_from_bits(g["h"]))
    hq_gpu = parity.decode_act(g["h"], g.get("h_scales"), s.act)
    zq_ref = rt["zq"] if s.latent_moe else mx.bf16_from_bits(wl.x_bits(T))
    clean_rows = ~zdirty[perm]
    hdirty_rows = np.zeros(T * s.k, bool)
    nh_el, n_el = 0, 0
    offsets = g["offsets"]
    for e in np.nonzero(g["counts"])[0]:
        r0, r1 = offsets[e], offsets[e + 1]
        rows = np.arange(r0, r1)[clean_rows[r0:r1]]
        if rows.size == 0:
            continue
        G, U, _ = (layer.dequant(m) for m in w.experts[e])
        h_ex, hb = parity.glu_hidden_bound(zq_ref[perm[rows]], G, U, layer.lora_factors(w, int(e), s),
                                           scaled_mfma=f8)
        err = np.abs(g["h_f32"][rows] - h_ex)
        assert np.all(err <= hb), f"expert {e}: hidden off by {np.max(err / hb):.3g} x the bound"
        diff = hq_gpu[rows] != rt["h"][rows]
        hdirty_rows[rows] = diff.any(axis=1)
        nh_el += int(diff.sum())
        n_el += diff.size
    nh = int(hdirty_rows.sum())
    # each differing code is a value within the bound above on the other side of a rounding boundary
    # (the encoder is checked strictly on the GPU's own values); they are rare among the elements
    assert nh_el <= max(2, 1e-3 * n_el), (nh_el, n_el)
    dirty = zdirty.copy()
    dirty[perm[hdirty_rows]] = True
    clean = ~dirty
    # each routed-path kernel against the oracle's step on the GPU's own (quantised) inputs
    sw = parity.stagewise(g, w, s, wl.x_bits(T))
    if s.Ns:
        parity.assert_y(mx.bf16_from_bits(g["hs"]), np.concatenate(rt["hs"], axis=1), "shared hidden")
    # the bar on y, every token: against the oracle whose quantisation decisions are taken on the GPU's
    # values (z and h after their quantisation points, strict-checked above against the oracle's encoder)
    zq_g = parity.decode_act(g["z"], g.get("z_scales"), s.act) if s.latent_moe else None
    hq_g = hq_gpu[g["inv"].reshape(T, s.k)]
    ref_q = layer.forward(wl.x_bits(T), w, s, select_override={t: gidx[t] for t in range(T)},
                          z_override=zq_g, h_override=hq_g)
    rel, ma = parity.assert_y(g["y"], ref_q.y)
    # and the same bar against the oracle's own chain on every token whose quantised activations all
    # equal the oracle's (most tokens; the rest differ by a code across a rounding boundary)
    # (the boundary codes themselves are bounded per element above; with wide rows a token often holds one)
    assert clean.sum() >= min(T // 8, 16), f"only {clean.sum()} of {T} tokens without a boundary code"
    rel_c, ma_c = float("nan"), float("nan")
    if clean.any():
        rel_c, ma_c = parity.assert_y(g["y"][clean], ref.y[clean], "y (oracle chain, clean tokens)")
        parity.assert_y(g["u"][clean], rt["u"][clean], "u (oracle chain, clean tokens)")
    if not f8:
        parity.assert_y(g["y"], ref.y, "y (oracle chain, every token)")
    _log(f"[check] {name} T={T}: flips {flips}, boundary codes z {int(zdirty.sum())} tokens / h {nh} rows "
         f"({nh_el} of {n_el} elements), "
         f"clean tokens {int(clean.sum())}/{T}; y vs oracle(GPU codes) rel_l2 {rel:.2e} maxabs/rms {ma:.2e}; "
         f"clean tokens vs oracle rel_l2 {rel_c:.2e} maxabs/rms {ma_c:.2e}; stagewise {sw}")
    return g


@pytest.mark.parametrize("name", ["tiny", "tiny_mxfp8", "tiny_mxfp8_many", "tiny_mxfp8_deep", "tiny_dense_many",
                                  "tiny_fullwidth", "tiny_skewed", "tiny_bf16_many", "tiny_bf16_deep", "tiny_split",
                                  "tiny_split_mxfp8", "tiny_e12_mxfp8", "tiny_e4_bf16", "tiny_lora",
                                  "tiny_lora_mxfp8_many", "tiny_lora_bf16_many", "tiny_lora_split",
                                  "tiny_lora_r32_skewed", "tiny_lora_mxfp8_r8"])
def test_full_parity(name):
    check_all(name, workloads.get(name).T)


@pytest.mark.parametrize("T", [1, 3, 16, 17, 40, 63])
def test_ragged_token_counts(T):
    check_all("tiny", T)


@pytest.mark.parametrize("T", [1, 17, 31])
def test_lora_ragged(T):
    """LoRA deltas on the panel kernel at ragged batch sizes (one row to two row tiles per expert)."""
    check_all("tiny_lora", T)


def test_mxfp8_ragged():
    check_all("tiny_mxfp8", 23)


@pytest.mark.parametrize("T", [129, 333, 511])
def test_mxfp8_many_rows_ragged(T):
    """Scaled-MFMA grouped kernel: expert row counts that leave partial 16-row tiles and chunks."""
    check_all("tiny_mxfp8_many", T)


@pytest.mark.parametrize("T", [1, 255, 777])
def test_mxfp8_deep_ragged(T):
    """Scaled-MFMA grouped kernel over several K windows and several 256-row chunks per expert."""
    check_all("tiny_mxfp8_deep", T)


@pytest.mark.parametrize("T", [129, 333, 511])
def test_bf16_many_rows_ragged(T):
    """Row-tiled grouped bf16 kernel: expert row counts that leave partial 16-row tiles and chunks."""
    check_all("tiny_bf16_many", T)


@pytest.mark.parametrize("T", [1, 255, 777])
def test_bf16_deep_ragged(T):
    """Row-tiled grouped bf16 kernel over several K windows and several 128-row chunks per expert
    (T = 1: the panel kernel alone)."""
    check_all("tiny_bf16_deep", T)


@pytest.mark.parametrize("name", ["tiny_split", "tiny_split_mxfp8"])
@pytest.mark.parametrize("T", [63, 64, 100])
def test_split_by_rows_ragged(name, T):
    """8 to 32 rows per expert on average: experts with 32 or more rows on the row-tiled kernel, the
    rest on the panel kernel, in the same stage (T = 63: the panel kernel alone)."""
    check_all(name, T)


@pytest.mark.parametrize("name", ["tiny_e4_all", "tiny_e4_all_mxfp8"])
@pytest.mark.parametrize("T", [15, 16, 17, 63, 64, 65, 127, 128])
def test_row_band_boundaries(name, T):
    """Every token chooses every one of the 4 experts, so each expert has exactly T rows: 15 rows (panel
    kernel), 16, 17 and 63 (mid-row kernel, one to four tiles), 64 and more (row-tiled kernels), and the
    switch that leaves the mid-row kernel unlaunched (T k = 128 E)."""
    check_all(name, T)


@pytest.mark.parametrize("T", [700, 1024, 1500])
def test_dense_many_rows_ragged(T):
    """Row-tiled dense GEMMs with a partial last chunk: 64-row chunks dealt panel block first (T = 700),
    128-row chunks dealt chunk first (T >= 1024)."""
    check_all("tiny_dense_many", T)


def test_deterministic_and_stream_order():
    wl, w, moe = case("tiny")
    x = workloads.device.x_tensor(wl)
    y1 = moe.forward(x)
    y2 = moe.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_identical_experts_gpu():
    """All experts equal: the routed branch equals one expert's output regardless of routing."""
    wl = workloads.get("tiny")
    w = ArrayWeights(wl)
    w.experts = [w.experts[2]] * wl.shape.E
    moe = workloads.device.build_layer(w, wl.shape, max_tokens=wl.T)
    g = run_gpu(moe, wl, wl.T)
    ref = layer.forward(wl.x_bits(), w, wl.shape)
    parity.assert_y(g["u"], ref.taps["u"], "u")
    parity.assert_y(g["y"], ref.y)


def test_t_zero_is_noop():
    wl, w, moe = case("tiny")
    x = torch.zeros(0, wl.shape.d, dtype=torch.bfloat16, device="cuda")
    y = moe.forward(x)
    assert y.shape == (0, wl.shape.d)


def test_too_many_tokens_rejected():
    wl, w, moe = case("tiny")
    x = workloads.device.x_tensor(wl.with_tokens(wl.T + 1))
    with pytest.raises(Exception) as ei:
        moe.forward(x)
    assert "max_tokens" in str(ei.value)

"""Pins of the oracle's layer forward against what the pages and the mathematics fix.

Each test names the passage it pins. Source pages: Kimi K3 course lesson 6
"LatentMoE" (eq. 11, eq. 13, "Deriving the headline number", table "What scales
with what") and "Serving K3, 01 architecture".
"""
import itertools
import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import layer, mx
from tests.weightset import ArrayWeights, identity_mxfp4, zero_mxfp4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))
TINY = workloads.get("tiny")


@pytest.fixture(scope="module")
def tiny_w():
    return ArrayWeights(TINY)


@pytest.fixture(scope="module")
def tiny_x():
    return TINY.x_bits()


def _near(v, g):
    return abs(v - g["value"]) <= g.get("rounding", 0)


# ---------------------------------------------------------------------------------------------
# closed forms printed on the pages
# ---------------------------------------------------------------------------------------------

def test_page_parameter_counts_from_workload_shapes():
    """lesson 6 'Deriving the headline number': 3 x 3584 x 3072 = 33.0M per expert, x 896 = 29.6B,
    x 92 layers = 2.72T; projections 4.7B and shared 12.2B over 92 layers; 16 active = 48.6B."""
    s = workloads.get("k3_decode_t64").shape
    per_expert = 2 * s.h * s.l + s.l * s.h            # gate [h,l] + up [h,l] + down [l,h]
    assert per_expert == 33_030_144
    assert _near(per_expert, GOLD["params_per_routed_expert"])
    pool = per_expert * s.E
    assert pool == 29_595_009_024 and _near(pool, GOLD["routed_pool_per_layer"])
    L = GOLD["moe_layers"]["value"]
    assert _near(pool * L, GOLD["routed_pool_all_layers"])
    assert _near(2 * s.d * s.l * L, GOLD["projections_all_layers"])
    assert _near(3 * s.d * s.hs * s.Ns * L, GOLD["shared_all_layers"])
    assert _near(s.k * per_expert * L, GOLD["active_routed_all_layers"])
    assert s.E // s.k == GOLD["sparsity_ratio"]["value"]
    # MXFP4 bytes of the resident routed pool: half a byte per element plus one scale byte per 32
    assert pool // 2 + pool // 32 == 15_722_348_544


def test_page_dispatch_payload():
    """lesson 6 table 'What scales with what': dispatch traffic k x 7168 = 114,688 at full width
    vs k x 3584 = 57,344 latent. Counted from the oracle's dispatched rows."""
    rng = np.random.default_rng(0)
    for name, gold in (("k3_decode_t64", GOLD["dispatch_latent"]), ("fullwidth_t64", GOLD["dispatch_full_width"])):
        s = workloads.get(name).shape
        k = 16                                        # the table compares at top-16
        T = 8
        idx = np.stack([rng.choice(s.E, k, replace=False) for _ in range(T)])
        counts, offsets, perm, inv = layer.routing_tables(idx, s.E)
        assert len(perm) == T * k
        assert len(perm) * s.expert_in == T * gold["value"]


def test_fullwidth_topk8_same_payload_as_latent_top16():
    """Serving article: top-16 latent costs what top-8 full width would (same bandwidth budget)."""
    lat = workloads.get("k3_decode_t64").shape
    full = workloads.get("fullwidth_t64").shape
    assert lat.k * lat.expert_in == full.k * full.expert_in == 57_344


# ---------------------------------------------------------------------------------------------
# router, eq. 13
# ---------------------------------------------------------------------------------------------

def test_p_sums_to_one(tiny_w, tiny_x):
    r = layer.forward(tiny_x, tiny_w, TINY.shape)
    p = r.taps["p"]
    assert np.all(p > 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-15


def test_topk_brute_force_tiny(tiny_w, tiny_x):
    """argtopk on the tiny layer equals the subset maximising the summed key, enumerated."""
    r = layer.forward(tiny_x, tiny_w, TINY.shape)
    key = r.taps["selection"].key
    E, k = TINY.shape.E, TINY.shape.k
    subsets = np.array(list(itertools.combinations(range(E), k)))
    assert len(subsets) == 1820
    for t in range(key.shape[0]):
        best = subsets[np.argmax(key[t][subsets].sum(axis=1))]
        got = r.taps["idx"][t]
        assert set(got.tolist()) == set(best.tolist())
        assert np.all(np.diff(key[t][got]) <= 0)          # rank order: descending key


def test_topk_tie_breaks_to_lower_id():
    s = np.array([[0.5, 0.7, 0.7, 0.1, 0.7]])
    sel = layer.select_topk(s, np.zeros(5), 2)
    assert sel.idx.tolist() == [[1, 2]]
    sel = layer.select_topk(s, np.zeros(5), 3)
    assert sel.idx.tolist() == [[1, 2, 4]]


def test_bias_steers_selection_not_weights(tiny_w, tiny_x):
    """eq. 13: b enters argtopk only; p is renormalised from s over the selected set."""
    w = tiny_w.copy()
    E = TINY.shape.E
    w.bias = np.zeros(E, np.float32)
    w.bias[5] = 100.0                                    # forces expert 5 for every token
    w.bias[9] = 50.0
    r = layer.forward(tiny_x, w, TINY.shape)
    idx, s, p = r.taps["idx"], r.taps["scores"], r.taps["p"]
    assert np.all(idx[:, 0] == 5) and np.all(idx[:, 1] == 9)
    ss = np.take_along_axis(s, idx, axis=1)
    assert np.allclose(p, ss / ss.sum(axis=1, keepdims=True), rtol=0, atol=1e-15)
    key = ss + w.bias[idx]
    assert not np.allclose(p, key / key.sum(axis=1, keepdims=True))
    # scores themselves do not depend on b
    r0 = layer.forward(tiny_x, tiny_w, TINY.shape)
    assert np.array_equal(r0.taps["scores"], s)


def test_router_matches_torch(tiny_w, tiny_x):
    xh = torch.from_numpy(mx.bf16_from_bits(tiny_x))
    Wr = torch.from_numpy(layer.dequant(tiny_w.w_router()))
    ref = torch.sigmoid(F.linear(xh, Wr)).numpy()
    r = layer.forward(tiny_x, tiny_w, TINY.shape)
    assert np.allclose(r.taps["scores"], ref, rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------------------------
# dispatch tables
# ---------------------------------------------------------------------------------------------

def test_routing_tables_invariants(tiny_w, tiny_x):
    r = layer.forward(tiny_x, tiny_w, TINY.shape)
    idx, counts, offsets, perm, inv = (r.taps[k] for k in ("idx", "counts", "offsets", "perm", "inv"))
    T, k = idx.shape
    assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
    for e in range(TINY.shape.E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                   # ascending token inside each segment
        assert set(seg.tolist()) == set(np.nonzero((idx == e).any(axis=1))[0].tolist())
    for t in range(T):
        for j in range(k):
            row = inv[t, j]
            assert perm[row] == t
            assert offsets[idx[t, j]] <= row < offsets[idx[t, j] + 1]
    assert sorted(inv.reshape(-1).tolist()) == list(range(T * k))


# ---------------------------------------------------------------------------------------------
# experts, combine, RMSNorm, shared: library special cases and invariants
# ---------------------------------------------------------------------------------------------

def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _bf16(v):
    return _t(mx.bf16_round(v.numpy()))


def test_identical_experts_degenerate_to_one_expert(tiny_w, tiny_x):
    """All experts equal => sum_i p_i E_i(z) = E(z) since sum p = 1 (eq. 11)."""
    w = tiny_w.copy()
    w.experts = [w.experts[3]] * TINY.shape.E
    r = layer.forward(tiny_x, w, TINY.shape)
    G, U, D = (layer.dequant(m) for m in w.experts[0])
    zq = _t(r.taps["zq"])
    h = _bf16(F.silu(F.linear(zq, _t(G))) * F.linear(zq, _t(U)))
    single = F.linear(h, _t(D)).numpy()
    assert np.allclose(r.taps["u"], single, rtol=1e-12, atol=1e-14)


def test_full_soft_mixture_when_k_equals_E(tiny_w, tiny_x):
    """k = E: every expert runs and u = sum_e (s_e / sum s) E_e(z); pins the pairing of p with outputs."""
    shape = replace(TINY.shape, k=TINY.shape.E)
    r = layer.forward(tiny_x, tiny_w, shape)
    s = _t(r.taps["scores"])
    p = s / s.sum(dim=1, keepdim=True)
    zq = _t(r.taps["zq"])
    u = torch.zeros(zq.shape[0], TINY.shape.l, dtype=torch.float64)
    for e in range(TINY.shape.E):
        G, U, D = (_t(layer.dequant(m)) for m in tiny_w.experts[e])
        h = _bf16(F.silu(F.linear(zq, G)) * F.linear(zq, U))
        u += p[:, e:e + 1] * F.linear(h, D)
    assert np.allclose(r.taps["u"], u.numpy(), rtol=1e-12, atol=1e-14)


def test_single_expert_layer_matches_torch(tiny_w, tiny_x):
    """E = 1, k = 1, no shared experts: y = W_up RMSNorm(E(W_down x)) (eq. 11), via torch fp64."""
    shape = replace(TINY.shape, E=1, k=1, Ns=0)
    w = tiny_w.copy()
    w.experts = w.experts[:1]
    w.bias = w.bias[:1]
    w.mats["w_router"] = (w.mats["w_router"][0][:1], w.mats["w_router"][1][:1])
    r = layer.forward(tiny_x, w, shape)
    x = _t(mx.bf16_from_bits(tiny_x))
    z = _bf16(F.linear(x, _t(layer.dequant(w.w_down()))))
    G, U, D = (_t(layer.dequant(m)) for m in w.experts[0])
    o = F.linear(_bf16(F.silu(F.linear(z, G)) * F.linear(z, U)), D)
    n = _bf16(F.rms_norm(o, (shape.l,), weight=_t(w.gamma), eps=shape.eps))
    y = F.linear(n, _t(layer.dequant(w.w_up()))).numpy()
    assert np.allclose(r.y, y, rtol=1e-12, atol=1e-13)
    assert np.all(r.taps["p"] == 1.0)


def test_shared_only_when_routed_experts_are_zero(tiny_w, tiny_x):
    """Zero routed experts => u = 0, RMSNorm(0) = 0, y = sum of shared experts on raw x (torch fp64)."""
    w = tiny_w.copy()
    s = TINY.shape
    z = (zero_mxfp4(s.h, s.l), zero_mxfp4(s.h, s.l), zero_mxfp4(s.l, s.h))
    w.experts = [z] * s.E
    r = layer.forward(tiny_x, w, s)
    x = _t(mx.bf16_from_bits(tiny_x))
    y = torch.zeros(x.shape[0], s.d, dtype=torch.float64)
    for j in range(s.Ns):
        G, U, D = (_t(layer.dequant(m)) for m in w.shared_mats[j])
        y += F.linear(_bf16(F.silu(F.linear(x, G)) * F.linear(x, U)), D)
    assert np.all(r.taps["u"] == 0)
    assert np.allclose(r.y, y.numpy(), rtol=1e-12, atol=1e-13)


def test_rmsnorm_scale_invariance(tiny_w, tiny_x):
    """lesson 6 'What extreme sparsity breaks': RMSNorm sits between aggregation and W_up, so
    doubling every routed expert output (+1 on each down-projection E8M0 scale) leaves y
    unchanged up to the eps term."""
    w2 = tiny_w.copy()
    w2.experts = [(g, u, (d[0], d[1] + 1)) for (g, u, d) in w2.experts]
    r1 = layer.forward(tiny_x, tiny_w, TINY.shape)
    r2 = layer.forward(tiny_x, w2, TINY.shape)
    assert np.array_equal(r2.taps["u"], 2 * r1.taps["u"])
    n1, n2 = r1.taps["n_pre"], r2.taps["n_pre"]
    eps = TINY.shape.eps
    ms = np.mean(r1.taps["u"] ** 2, axis=1, keepdims=True)
    ratio = np.sqrt((ms + eps) / (ms + eps / 4))          # closed form of the eps effect
    assert np.allclose(n2, n1 * ratio, rtol=1e-13, atol=0)
    assert np.max(np.abs(ratio - 1)) < eps / ms.min()
    # y moves only where the bf16 rounding of n lands on the other side of a midpoint
    rel = np.linalg.norm(r2.y - r1.y) / np.linalg.norm(r1.y)
    assert rel < 1e-3
    # and the routed branch is not a no-op: dropping it changes y a lot
    assert np.linalg.norm(r1.taps["y_routed"]) > 0.1 * np.linalg.norm(r1.y)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(5)
    u = rng.normal(size=(7, 96)) * 3
    g = rng.normal(size=96)
    ref = F.rms_norm(_t(u), (96,), weight=_t(g), eps=1e-6).numpy()
    assert np.allclose(layer.rmsnorm(u, g, 1e-6), ref, rtol=1e-14, atol=1e-15)


def test_identity_projections_reduce_to_conventional_moe(tiny_w, tiny_x):
    """l = d with W_down = W_up = I: the latent layer is the conventional full-width MoE with
    an RMSNorm on the routed sum (lesson 6: LatentMoE differs by the projections + RMSNorm)."""
    s = TINY.shape
    d = s.d
    lat = replace(s, l=d)
    full = replace(s, l=d, latent_moe=0)
    wl = workloads.Workload("tiny_id", full, T=16, seed=7)
    w = ArrayWeights(wl)
    w.mats["w_down"] = identity_mxfp4(d)
    w.mats["w_up"] = identity_mxfp4(d)
    w.gamma = np.ones(d, np.float32)
    x = TINY.x_bits()[:16]
    rl = layer.forward(x, w, lat)
    rf = layer.forward(x, w, full)
    assert np.array_equal(rl.taps["idx"], rf.taps["idx"])
    routed_full = rf.y - rf.taps["y_shared"]
    expect = mx.bf16_round(layer.rmsnorm(routed_full, w.gamma, s.eps))
    assert np.allclose(rl.y - rl.taps["y_shared"], expect, rtol=1e-12, atol=1e-13)


def test_mxfp8_activation_points(tiny_w, tiny_x):
    """'mxfp8' workloads: the routed GEMM inputs z and h are MXFP8 values (decode exactly from
    their codes), everything else as in the bf16 workload."""
    shape = replace(TINY.shape, act="mxfp8")
    r = layer.forward(tiny_x, tiny_w, shape)
    assert np.array_equal(mx.mx_dequantize(r.taps["z_codes"], r.taps["z_scales"], "e4m3"), r.taps["zq"])
    c, sb = mx.mx_quantize(r.taps["hpre"], "e4m3")
    assert np.array_equal(mx.mx_dequantize(c, sb, "e4m3"), r.taps["h"])
    rb = layer.forward(tiny_x, tiny_w, TINY.shape)
    rel = np.linalg.norm(r.y - rb.y) / np.linalg.norm(rb.y)
    assert 0 < rel < 0.05                                   # same layer, coarser activations


def test_select_override_and_flip_check(tiny_w, tiny_x):
    r = layer.forward(tiny_x, tiny_w, TINY.shape)
    sel = r.taps["selection"]
    ok, flip = layer.check_selection(r.taps["idx"], sel)
    assert ok.all() and not flip.any()
    bad = r.taps["idx"].copy()
    bad[0, [0, 1]] = bad[0, [1, 0]]                         # order swap with a real gap
    ok, flip = layer.check_selection(bad, sel)
    assert not ok[0] and ok[1:].all()
    ok, flip = layer.check_selection(bad, sel, tol=1.0)     # inside a (huge) tolerance: a flip
    assert ok[0] and flip[0]
    r2 = layer.forward(tiny_x, tiny_w, TINY.shape, select_override={0: bad[0]})
    assert np.allclose(r2.y[1:], r.y[1:]) and np.allclose(r2.y[0], r.y[0])   # same set, same y


def test_generator_weights_are_oracle_mx_encoding():
    """The workload generator's MXFP4 weights equal the oracle's MX encoding of the same fp32
    normals (ties the generator's encoder to the pinned codec)."""
    N, K, std = 8, 256, 256 ** -0.5
    codes, scales = workloads.mxfp4(11, workloads.GATE, 3, N, K, std)
    vals = workloads.normal(11, workloads.GATE, 3, (N, K), std).astype(np.float64)
    c2, s2 = mx.mx_quantize(vals, "e2m1")
    assert np.array_equal(scales, s2)
    assert np.array_equal(mx.unpack_fp4(codes), c2)


# ---------------------------------------------------------------------------------------------
# the override path (activations after their quantisation points supplied from outside)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_override_with_own_quantised_values_is_identity(tiny_w, tiny_x, act):
    """z_override / h_override fed with the oracle's own quantised z and hidden (the hidden given per
    (token, selection slot)) reproduce the oracle's own output bit for bit."""
    shape = replace(TINY.shape, act=act)
    r = layer.forward(tiny_x, tiny_w, shape)
    h_tk = r.taps["h"][r.taps["inv"]]                       # dispatched rows -> [T, k, h]
    r2 = layer.forward(tiny_x, tiny_w, shape, z_override=r.taps["zq"], h_override=h_tk)
    assert np.array_equal(r2.y, r.y)
    assert np.array_equal(r2.taps["expert_out"], r.taps["expert_out"])
    assert np.array_equal(r2.taps["u"], r.taps["u"])


@pytest.mark.parametrize("t,j", [(0, 0), (3, 1), (17, 3), (63, 2)])
def test_override_hidden_lands_on_its_token_and_slot(tiny_w, tiny_x, t, j):
    """A one-hot hidden at (token t, slot j) and zeros elsewhere: the combine gives u_t = p_tj times
    column m of the down-projection of expert idx[t, j] (eq. 11), and u = 0 for every other token.
    Fixes the dispatched-row <-> (token, slot) mapping of the override path by construction."""
    s = TINY.shape
    r = layer.forward(tiny_x, tiny_w, s)
    T = tiny_x.shape[0]
    m = 5 + 7 * j
    h = np.zeros((T, s.k, s.h))
    h[t, j, m] = 1.0
    r2 = layer.forward(tiny_x, tiny_w, s, z_override=r.taps["zq"], h_override=h)
    e = r.taps["idx"][t, j]
    D = layer.dequant(tiny_w.experts[e][2])
    expect = r.taps["p"][t, j] * D[:, m]
    assert np.array_equal(r2.taps["u"][t], expect)
    others = np.arange(T) != t
    assert np.all(r2.taps["u"][others] == 0)


def test_override_z_row_feeds_its_token_only(tiny_w, tiny_x):
    """Changing the overriding latent of one token changes that token's routed branch only."""
    s = TINY.shape
    r = layer.forward(tiny_x, tiny_w, s)
    zq = r.taps["zq"].copy()
    zq[9] = zq[10]
    r2 = layer.forward(tiny_x, tiny_w, s, z_override=zq)
    keep = np.arange(tiny_x.shape[0]) != 9
    assert np.array_equal(r2.y[keep], r.y[keep])
    assert not np.allclose(r2.y[9], r.y[9])


# ---------------------------------------------------------------------------------------------
# where MXFP8 mode quantises (and where it does not)
# ---------------------------------------------------------------------------------------------

def _mantissa_bits_needed(v):
    """Fraction bits of each nonzero value beyond its leading one (exact for fp64 inputs)."""
    a = np.abs(v[v != 0])
    m, _ = np.frexp(a)                                      # a = m 2^e, m in [0.5, 1)
    bits = np.zeros(a.shape, np.int64)
    f = m * 2.0 - 1.0                                       # fraction in [0, 1)
    for b in range(1, 60):
        f = f * 2.0
        one = f >= 1.0
        f = np.where(one, f - 1.0, f)
        bits = np.where(f > 0, b + 1, bits)
    return bits


def test_mxfp8_mode_quantises_only_z_and_h(tiny_w, tiny_x):
    """MXFP8 workloads put MX quantisation at the routed GEMM inputs only (the workload definition:
    the latent and the hidden fed to the grouped GEMMs). The shared experts' path is the bf16 one
    unchanged, the RMSNorm output is the bf16 rounding of RMSNorm(u) (torch fp64 reference) on the
    run's own u, and neither carries values off the bf16 grid nor is restricted to 3 mantissa bits."""
    s8 = replace(TINY.shape, act="mxfp8")
    r8 = layer.forward(tiny_x, tiny_w, s8)
    rb = layer.forward(tiny_x, tiny_w, TINY.shape)
    # shared path: identical to the bf16 workload's
    assert all(np.array_equal(a, b) for a, b in zip(r8.taps["hs"], rb.taps["hs"]))
    assert np.array_equal(r8.taps["y_shared"], rb.taps["y_shared"])
    # latent before quantisation: the same W_down x; after: its MX encoding, not its bf16 rounding
    assert np.array_equal(r8.taps["z"], rb.taps["z"])
    assert not np.array_equal(r8.taps["zq"], rb.taps["zq"])
    assert _mantissa_bits_needed(r8.taps["zq"]).max() <= 3
    # n: bf16 rounding of RMSNorm of this run's u
    ref = F.rms_norm(_t(r8.taps["u"]), (s8.l,), weight=_t(tiny_w.gamma), eps=s8.eps).numpy()
    assert np.array_equal(r8.taps["n"], mx.bf16_round(ref))
    assert _mantissa_bits_needed(r8.taps["n"]).max() > 3
    assert _mantissa_bits_needed(np.concatenate(r8.taps["hs"], axis=1)).max() > 3
    # the hidden fed to the down-projection: MX values (at most 3 mantissa bits)
    assert _mantissa_bits_needed(r8.taps["h"]).max() <= 3

"""Pins of the oracle's BF16 LoRA deltas over the MXFP4 experts ("Serving K3, 01 architecture", the
paragraph on the MXFP4 KL floor: fine-tuning ships BF16 LoRA deltas over the 4-bit base weights).
Reading: every routed expert matrix W becomes W + B A (bf16 A [r, K], B [N, r]), applied as B (A v).
Pinned by what that fixes: zero deltas change nothing; a delta equal to a known edit of the base
weights reproduces the layer with those weights edited; experts that are all equal (deltas included)
degenerate to one expert; the result equals the merged fp64 weights W + B A."""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest

import workloads
from oracle import layer, mx
from tests.weightset import ArrayWeights

WL = workloads.get("tiny_lora")
S = WL.shape


@pytest.fixture(scope="module")
def w():
    return ArrayWeights(WL)


@pytest.fixture(scope="module")
def x():
    return WL.x_bits()


def _bits(a):
    return mx.bf16_to_bits(a)


def _with_loras(w, loras):
    w2 = w.copy()
    w2.loras = loras
    return w2


def test_lora_delta_is_not_negligible(w, x):
    """The workload's deltas move the routed branch (else the GPU parity tests would not see them)."""
    r = layer.forward(x, w, S)
    r0 = layer.forward(x, w, replace(S, lora_rank=0))
    rel = np.linalg.norm(r.taps["u"] - r0.taps["u"]) / np.linalg.norm(r0.taps["u"])
    assert 0.05 < rel < 1.0, rel


def test_zero_deltas_change_nothing(w, x):
    zero = [{k: np.zeros_like(v) for k, v in lo.items()} for lo in w.loras]
    r = layer.forward(x, _with_loras(w, zero), S)
    r0 = layer.forward(x, w, replace(S, lora_rank=0))
    assert np.array_equal(r.y, r0.y)


@pytest.mark.parametrize("mat", ["gate", "up", "down"])
def test_delta_equal_to_a_weight_edit(w, x, mat):
    """A rank-1 delta B A with B = e_i (one 1 in column 0) and A = row i of the dequantised base matrix
    doubles that row: the layer equals the one whose MXFP4 row i has every E8M0 scale raised by one
    (exactly x2), with no deltas. Fixes where each factor enters (which matrix, B A not A B, the sign)."""
    i = 7
    e_mod = list(range(S.E))
    loras = []
    for e in e_mod:
        G, U, D = (layer.dequant(m) for m in w.experts[e])
        base = {"gate": G, "up": U, "down": D}[mat]
        N, K = base.shape
        lo = {k: np.zeros_like(v) for k, v in w.loras[e].items()}
        A = np.zeros((S.lora_rank, K))
        A[0] = base[i]
        B = np.zeros((N, S.lora_rank))
        B[i, 0] = 1.0
        assert np.array_equal(mx.bf16_round(A), A)          # MXFP4 values are exact in bf16
        lo["a_" + mat] = _bits(A)
        lo["b_" + mat] = _bits(B)
        loras.append(lo)
    r = layer.forward(x, _with_loras(w, loras), S)
    w2 = w.copy()
    idx = {"gate": 0, "up": 1, "down": 2}[mat]
    ex = []
    for e in range(S.E):
        mats = list(w.experts[e])
        c, sc = mats[idx]
        sc = sc.copy()
        sc[i] += 1
        mats[idx] = (c, sc)
        ex.append(tuple(mats))
    w2.experts = ex
    r2 = layer.forward(x, w2, replace(S, lora_rank=0))
    assert np.allclose(r.taps["u"], r2.taps["u"], rtol=1e-12, atol=1e-13)
    assert np.allclose(r.y, r2.y, rtol=1e-12, atol=1e-12)
    # and the edit is not a no-op
    r0 = layer.forward(x, w, replace(S, lora_rank=0))
    assert not np.allclose(r.taps["u"], r0.taps["u"], rtol=1e-6)


def test_identical_experts_and_deltas_degenerate_to_one_expert(w, x):
    """All experts (and their deltas) equal: u = E'(z) for the single expert E' with its deltas (eq. 11,
    sum p = 1), computed with merged fp64 weights W + B A."""
    w2 = w.copy()
    w2.experts = [w.experts[5]] * S.E
    w2.loras = [w.loras[5]] * S.E
    r = layer.forward(x, w2, S)
    lo = {k: mx.bf16_from_bits(v) for k, v in w.loras[5].items()}
    G, U, D = (layer.dequant(m) for m in w.experts[5])
    Gm, Um, Dm = G + lo["b_gate"] @ lo["a_gate"], U + lo["b_up"] @ lo["a_up"], D + lo["b_down"] @ lo["a_down"]
    z = r.taps["zq"]
    h = mx.bf16_round(layer.silu(z @ Gm.T) * (z @ Um.T))
    assert np.allclose(r.taps["u"], h @ Dm.T, rtol=1e-10, atol=1e-12)


def test_matches_merged_weights_per_expert(w, x):
    """Every dispatched row: the expert output equals the fp64 GLU with merged weights W + B A."""
    r = layer.forward(x, w, S)
    perm, offsets = r.taps["perm"], r.taps["offsets"]
    for e in np.nonzero(r.taps["counts"])[0]:
        lo = {k: mx.bf16_from_bits(v) for k, v in w.loras[e].items()}
        G, U, D = (layer.dequant(m) for m in w.experts[e])
        z = r.taps["zq"][perm[offsets[e]:offsets[e + 1]]]
        hpre = layer.silu(z @ (G + lo["b_gate"] @ lo["a_gate"]).T) * (z @ (U + lo["b_up"] @ lo["a_up"]).T)
        assert np.allclose(r.taps["hpre"][offsets[e]:offsets[e + 1]], hpre, rtol=1e-11, atol=1e-13)
        o = r.taps["h"][offsets[e]:offsets[e + 1]] @ (D + lo["b_down"] @ lo["a_down"]).T
        assert np.allclose(r.taps["expert_out"][offsets[e]:offsets[e + 1]], o, rtol=1e-11, atol=1e-13)


def test_shared_and_router_untouched_by_deltas(w, x):
    r = layer.forward(x, w, S)
    r0 = layer.forward(x, w, replace(S, lora_rank=0))
    assert np.array_equal(r.taps["scores"], r0.taps["scores"])
    assert np.array_equal(r.taps["y_shared"], r0.taps["y_shared"])
    assert np.array_equal(r.taps["zq"], r0.taps["zq"])

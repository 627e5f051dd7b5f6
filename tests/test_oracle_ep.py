"""Pins of the oracle's expert-parallel send side ("Serving K3, 01 architecture": experts sharded over
accelerators with an all-to-all of data-dependent sizes; "Kimi K3: architectural innovations",
"Compress the expert interface": the latent is what crosses; lesson 6, table "What scales with what":
k x 3584 = 57,344 values per token). Experts in n_ranks contiguous ranges."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import workloads
from oracle import layer
from tests.weightset import ArrayWeights

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_send_counts_brute_force():
    rng = np.random.default_rng(0)
    T, E, k = 37, 24, 5
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    for n in (1, 2, 3, 4, 6, 8, 12, 24):
        got = layer.ep_send_counts(idx, E, n)
        per = E // n
        brute = [sum(1 for t in range(T) for j in range(k) if idx[t, j] // per == r) for r in range(n)]
        assert got.tolist() == brute
        assert got.sum() == T * k
    counts, offsets, perm, inv = layer.routing_tables(idx, E)
    assert layer.ep_send_counts(idx, E, E).tolist() == counts.tolist()
    # each rank's share is a contiguous run of the dispatched order
    got = layer.ep_send_counts(idx, E, 4)
    starts = np.concatenate([[0], np.cumsum(got)])
    for r in range(4):
        assert starts[r] == offsets[r * E // 4] and starts[r + 1] == offsets[(r + 1) * E // 4]


def test_send_payload_is_the_latent():
    """Per token the send buffer holds k rows of width l: 57,344 values at the K3 shape."""
    s = workloads.get("k3_decode_t64").shape
    T = 3
    rng = np.random.default_rng(1)
    idx = np.stack([rng.choice(s.E, s.k, replace=False) for _ in range(T)])
    counts, offsets, perm, inv = layer.routing_tables(idx, s.E)
    z = rng.normal(size=(T, s.l))
    rows = layer.ep_send_rows(z, perm)
    assert rows.size == T * GOLD["dispatch_latent"]["value"]
    for row, t in enumerate(perm):
        assert np.array_equal(rows[row], z[t])


def test_rank_shares_reassemble_the_layer():
    """Running each rank's experts on its share of the send rows and concatenating the outputs in send
    order gives the layer's own expert outputs (the experts of different ranks never share a row)."""
    wl = workloads.get("tiny")
    w = ArrayWeights(wl)
    s = wl.shape
    r = layer.forward(wl.x_bits(), w, s)
    send = layer.ep_send_rows(r.taps["zq"], r.taps["perm"])
    n = 4
    counts = layer.ep_send_counts(r.taps["idx"], s.E, n)
    starts = np.concatenate([[0], np.cumsum(counts)])
    per = s.E // n
    out = []
    for rk in range(n):
        rows = send[starts[rk]:starts[rk + 1]]
        loc = r.taps["counts"][rk * per:(rk + 1) * per]
        loff = np.concatenate([[0], np.cumsum(loc)])
        for i in range(per):
            G, U, D = (layer.dequant(m) for m in w.experts[rk * per + i])
            o, *_ = layer.glu(rows[loff[i]:loff[i + 1]], G, U, D, s.act)
            out.append(o)
    assert np.array_equal(np.concatenate(out), r.taps["expert_out"])


def test_send_counts_reject_uneven_ranges():
    with pytest.raises(AssertionError):
        layer.ep_send_counts(np.zeros((2, 2), np.int64), 10, 4)

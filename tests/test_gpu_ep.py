"""GPU parity of the expert-parallel split of the forward ("Serving K3, 01 architecture": expert
parallelism with an all-to-all of data-dependent sizes; "Kimi K3: architectural innovations",
"Compress the expert interface": the latent crosses the interconnect), on one GPU.

k3moe_forward_head on the full layer gives the send buffer (the routed input in dispatched order),
the rows per destination rank and the rows per expert; each rank's experts, packed into a context of
their own (E / n_ranks experts, no dense part), run on their share of the send buffer with
k3moe_experts_forward; k3moe_forward_tail combines the concatenated outputs at the origin. Checked:
send counts exact against the oracle's, the send buffer bit for bit against the latent gathered in
dispatched order, and the split forward's y bit-identical to k3moe_forward's (the same kernels on the
same rows), for bf16 and MXFP8 activations, the full-width layer and LoRA deltas. Shapes: the tiny
layers (16 experts over 2 or 4 ranks, 64 to 512 tokens)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads
import workloads.device as wdev
from oracle import layer
from tests.weightset import ArrayWeights

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.__stderr__, flush=True)


@pytest.mark.parametrize("name,n_ranks", [("tiny", 4), ("tiny", 2), ("tiny_mxfp8_many", 4), ("tiny_fullwidth", 2),
                                          ("tiny_lora", 4), ("tiny_lora_mxfp8_many", 2), ("tiny_split", 4)])
def test_split_forward_matches_forward(name, n_ranks):
    wl = workloads.get(name)
    s = wl.shape
    T = wl.T
    w = ArrayWeights(wl)
    full = wdev.build_layer(w, s, max_tokens=T)
    per = s.E // n_ranks
    ranks = [wdev.build_layer(w, s, max_tokens=T, experts=range(r * per, (r + 1) * per), dense=False)
             for r in range(n_ranks)]
    x = wdev.x_tensor(wl, T)
    idx = torch.empty(T, s.k, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * s.k, dtype=torch.int32, device="cuda")
    taps = {"topk_idx": idx, "perm": perm}
    f8 = s.act == "mxfp8" and s.latent_moe
    if s.latent_moe:
        taps["z"] = torch.empty(T, s.l, dtype=torch.uint8 if f8 else torch.bfloat16, device="cuda")
        if f8:
            taps["z_scales"] = torch.empty(T, s.l // 32, dtype=torch.uint8, device="cuda")
    y_ref = full.forward(x, taps=taps)
    rows, scales, send, counts = full.forward_head(x, n_ranks)
    torch.cuda.synchronize()
    # send side against the oracle's definitions
    send_np = send.cpu().numpy()
    assert send_np.tolist() == layer.ep_send_counts(idx.cpu().numpy(), s.E, n_ranks).tolist()
    assert counts.cpu().numpy().tolist() == np.bincount(idx.cpu().numpy().reshape(-1), minlength=s.E).tolist()
    src = taps["z"] if s.latent_moe else x
    pl = perm.cpu().long()
    assert torch.equal(rows.view(torch.uint8).cpu(), src.contiguous().view(torch.uint8).cpu()[pl])
    if f8:
        assert torch.equal(scales.cpu(), taps["z_scales"].cpu()[pl])
    # each rank on its share, outputs concatenated in send order, tail at the origin
    outs, start = [], 0
    for r in range(n_ranks):
        n = int(send_np[r])
        sl = slice(start, start + n)
        outs.append(ranks[r].experts_forward(rows[sl], scales[sl] if f8 else None,
                                             counts[r * per:(r + 1) * per].contiguous()))
        start += n
    O = torch.cat(outs)
    y = full.forward_tail(O, T)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    _log(f"[ep] {name} over {n_ranks} ranks: send counts {send_np.tolist()}, y bit-identical to the forward")


def test_head_with_no_tokens_sends_nothing():
    wl = workloads.get("tiny")
    full = wdev.build_layer(ArrayWeights(wl), wl.shape, max_tokens=wl.T)
    x = torch.zeros(0, wl.shape.d, dtype=torch.bfloat16, device="cuda")
    rows, scales, send, counts = full.forward_head(x, 4)
    torch.cuda.synchronize()
    assert send.cpu().tolist() == [0, 0, 0, 0] and int(counts.sum()) == 0


def test_experts_forward_clamps_to_the_rows_given():
    """Counts that claim more rows than were received: no row beyond R is read or written (the
    outputs of the rows that are there still match the full layer's)."""
    wl = workloads.get("tiny")
    s = wl.shape
    w = ArrayWeights(wl)
    full = wdev.build_layer(w, s, max_tokens=wl.T)
    loc = wdev.build_layer(w, s, max_tokens=wl.T, experts=range(0, 4), dense=False)
    x = wdev.x_tensor(wl)
    rows, _, send, counts = full.forward_head(x, 4)
    n = int(send[0])
    guard = torch.full((n + 64, s.l), 7.0, dtype=torch.float32, device="cuda")
    c = counts[:4].clone()
    c[3] += 1000                                          # more than was sent
    loc.experts_forward(rows[:n], None, c, out=guard[:n])
    torch.cuda.synchronize()
    assert torch.all(guard[n:] == 7.0)

"""GPU parity of the Quantile Balancing bias (k3moe_quantile_bias) against the oracle
(oracle/balance.py): the bias is a selection among the scores, so GPU and oracle agree bit for bit.
Sizes: tiny (E = 16, k = 4) up to the K3 router (E = 896, k = 16) over calibration batches of 1 to
16384 tokens, with ties; the error path for too large a batch; the calibrated bias applied to the
skewed tiny layer's own router scores."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import latent_width_expert_amd as lwe
import workloads
import workloads.device
from oracle import balance, layer
from tests.weightset import ArrayWeights

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _ctx(E, k):
    return lwe.K3MoE(lwe.LayerConfig(d_model=256, latent=128, hidden=128, n_experts=E, top_k=k, n_shared=1,
                                     shared_hidden=96, max_tokens=64))


@pytest.mark.parametrize("T,E,k,ties", [(1, 16, 4, False), (64, 16, 4, False), (777, 12, 3, True),
                                        (1000, 896, 16, False), (8192, 896, 16, False), (8192, 896, 16, True),
                                        (16384, 896, 16, False)])
def test_quantile_bias_bit_exact(T, E, k, ties):
    rng = np.random.default_rng(T + E)
    s = (rng.integers(1, 9, (T, E)) / 8.0 if ties else rng.random((T, E)) + 1e-3).astype(np.float32)
    moe = _ctx(E, k)
    sd = torch.from_numpy(s).cuda()
    b = moe.quantile_bias(sd)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    moe.quantile_bias(sd)
    ev1.record()
    torch.cuda.synchronize()
    ref = balance.quantile_bias(s, k)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    _log(f"[balance] T={T} E={E} k={k} ties={ties}: bit-exact, {ev0.elapsed_time(ev1) * 1e3:.1f} us")


def test_quantile_bias_rejects_large_batch():
    moe = _ctx(16, 4)
    s = torch.zeros(16385, 16, dtype=torch.float32, device="cuda")
    with pytest.raises(lwe.K3MoEError) as ei:
        moe.quantile_bias(s)
    assert "16384" in str(ei.value)


def test_calibrated_bias_balances_skewed_layer():
    """The skewed tiny layer (Zipf router bias): its GPU router scores over the batch give the
    calibrated bias; top-k loads with it have a smaller max/mean than with the layer's own bias."""
    wl = workloads.get("tiny_skewed")
    s_ = wl.shape
    w = ArrayWeights(wl)
    moe = workloads.device.build_layer(w, s_, max_tokens=wl.T)
    x = workloads.device.x_tensor(wl)
    scores = torch.empty(wl.T, s_.E, dtype=torch.float32, device="cuda")
    moe.forward(x, taps={"scores": scores})
    b = moe.quantile_bias(scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy().astype(np.float64)
    assert np.array_equal(b.cpu().numpy(), balance.quantile_bias(scores.cpu().numpy(), s_.k))

    def load(bias):
        c = np.bincount(layer.select_topk(sc, bias.astype(np.float64), s_.k).idx.reshape(-1), minlength=s_.E)
        return c.max() / c.mean()

    before, after = load(wl.router_bias()), load(b.cpu().numpy())
    _log(f"[balance] tiny_skewed: max/mean load {before:.2f} with the layer's bias, {after:.2f} calibrated")
    assert after < before

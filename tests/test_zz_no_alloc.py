"""The entry point that allocates nothing (k3moe_forward_noalloc, the library's static device scratch
in place of a workspace) against k3moe_forward with a workspace, through the C ABI: bit-identical
outputs (the same kernels on the same inputs) on two calls in a row, the second with fewer tokens,
and a batch whose workspace exceeds the scratch rejected before any device work. Tiny layers (bf16,
MXFP8, LoRA) and the K3-shape decode batch."""
from __future__ import annotations

import sys

import pytest
import torch

import latent_width_expert_amd as lwe
import workloads
import workloads.device as wdev
from tests.weightset import ArrayWeights

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.__stderr__, flush=True)


@pytest.mark.parametrize("name", ["tiny", "tiny_mxfp8_many", "tiny_lora", "k3_decode_t64"])
def test_noalloc_matches_forward(name):
    """(k3_decode_t64: the K3-shape decode batch of 64 tokens, whose workspace fits the scratch.)"""
    wl = workloads.get(name)
    prov = wl if name.startswith("k3") else ArrayWeights(wl)
    moe = wdev.build_layer(prov, wl.shape, max_tokens=wl.T)
    for T in (wl.T, wl.T // 2 - 3):
        x = wdev.x_tensor(wl, T)
        y_ref = moe.forward(x)
        y = torch.full_like(y_ref, float("nan"))
        assert moe.scratch_fits(T)
        moe.forward_noalloc(x, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (name, T)
        _log(f"[noalloc] {name} T={T}: bit-identical to the workspace forward")


def test_noalloc_rejects_batches_beyond_the_scratch():
    wl = workloads.get("tiny")
    moe = wdev.build_layer(ArrayWeights(wl), wl.shape, max_tokens=40000)
    T = 40000
    assert not moe.scratch_fits(T)
    x = torch.zeros(T, wl.shape.d, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(lwe.K3MoEError) as ei:
        moe.forward_noalloc(x, y)
    assert ei.value.code == lwe.ETOOBIG and "scratch" in str(ei.value)

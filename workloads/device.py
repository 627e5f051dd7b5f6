"""Put a workload's weights onto the GPU through the library's packer.

Test and benchmark infrastructure (not part of the library): it draws canonical MX tensors with
the seeded generator, uploads them with torch and hands them to `K3MoE.pack`. For K3-size pools
the routed experts are drawn on a background thread in chunks while the previous chunk is
uploaded and packed, so host memory holds a few chunks at most.
"""
from __future__ import annotations

import queue
import sys
import threading
import time

import numpy as np
import torch

from latent_width_expert_amd import K3MoE, LayerConfig

from . import Workload


def layer_config(shape, max_tokens: int, n_experts: int | None = None) -> LayerConfig:
    return LayerConfig(d_model=shape.d, latent=shape.l if shape.latent_moe else shape.d, hidden=shape.h,
                       n_experts=shape.E if n_experts is None else n_experts, top_k=shape.k, n_shared=shape.Ns,
                       shared_hidden=shape.hs, latent_moe=shape.latent_moe, act=shape.act, max_tokens=max_tokens,
                       rms_eps=shape.eps, lora_rank=shape.lora_rank)


def _lora_dev(stack, i, device):
    """One expert's LoRA factors (bf16 bit patterns) as bf16 device tensors."""
    return {n: torch.from_numpy(np.ascontiguousarray(v[i]).view(np.int16)).to(device).view(torch.bfloat16)
            for n, v in stack.items()}


def _dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _pair(p, device):
    return (_dev(p[0], device), _dev(p[1], device))


def _one(p):
    c, s = p
    return (c[0], s[0]) if c.ndim == 3 else (c, s)


def upload_dense(provider, shape, device="cuda"):
    dense = {"w_router": _pair(provider.w_router(), device),
             "router_bias": _dev(provider.router_bias().astype(np.float32), device)}
    if shape.latent_moe:
        dense["w_down"] = _pair(provider.w_down(), device)
        dense["w_up"] = _pair(provider.w_up(), device)
        dense["rms_gamma"] = _dev(provider.rms_gamma().astype(np.float32), device)
    dense["shared"] = [tuple(_pair(m, device) for m in provider.shared(j)) for j in range(shape.Ns)]
    return dense


def _log(msg):
    print(msg, file=sys.__stderr__, flush=True)


def build_layer(provider, shape, max_tokens: int, device="cuda", chunk: int = 32, verbose: bool = False,
                experts=None, dense: bool = True) -> K3MoE:
    """Create, allocate and pack a layer from a weight provider (a workloads.Workload or any
    object with the same accessors). Returns the packed K3MoE. experts: optional range of the
    provider's routed experts to hold (one expert-parallel rank's share; the context then has
    len(experts) experts); dense=False leaves the dense part unpacked (an expert-only rank)."""
    ex = range(shape.E) if experts is None else experts
    moe = K3MoE(layer_config(shape, max_tokens, n_experts=len(ex))).allocate(device)
    stream = torch.cuda.current_stream()
    if dense:
        dn = upload_dense(provider, shape, device)
        moe.pack(dense=dn)
        stream.synchronize()
        del dn
    E = len(ex)
    base = ex.start
    many = isinstance(provider, Workload) or getattr(provider, "chunked", False)
    lora = shape.lora_rank > 0

    def produce(q):
        for e0 in range(0, E, chunk):
            n = min(chunk, E - e0)
            g0 = base + e0
            if many:
                mats = provider.routed(g0, n)
                lo = provider.lora(g0, n) if lora else None
            else:
                ms = [provider.routed(e) for e in range(g0, g0 + n)]
                mats = tuple((np.stack([_one(m[i])[0] for m in ms]), np.stack([_one(m[i])[1] for m in ms]))
                             for i in range(3))
                los = [provider.lora(e) for e in range(g0, g0 + n)] if lora else None
                lo = {k: np.stack([m[k] for m in los]) for k in los[0]} if lora else None
            q.put((e0, mats, lo))
        q.put(None)

    q = queue.Queue(maxsize=2)
    th = threading.Thread(target=produce, args=(q,), daemon=True)
    t0 = time.time()
    th.start()
    while True:
        item = q.get()
        if item is None:
            break
        e0, (g, u, d), lo = item
        n = g[0].shape[0]
        gd, ud, dd = _pair(g, device), _pair(u, device), _pair(d, device)
        routed = [((gd[0][i], gd[1][i]), (ud[0][i], ud[1][i]), (dd[0][i], dd[1][i])) for i in range(n)]
        lod = [_lora_dev(lo, i, device) for i in range(n)] if lo is not None else None
        moe.pack(routed=routed, routed_first=e0, lora=lod)
        stream.synchronize()
        del gd, ud, dd, routed, lod
        if verbose and (e0 // chunk) % 8 == 0:
            _log(f"[pack] experts {e0 + n}/{E} ({time.time() - t0:.1f} s)")
    th.join()
    return moe


def x_tensor(wl, T=None, device="cuda"):
    bits = wl.x_bits(T)
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)

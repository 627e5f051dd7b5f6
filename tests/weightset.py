"""In-memory canonical MX weight sets for tests (materialised from a workload, editable)."""
from __future__ import annotations

import copy

import numpy as np


class ArrayWeights:
    """All canonical tensors of one layer held as numpy arrays.

    Matrices are (codes [N, K/2] uint8, scales [N, K/32] uint8) pairs; routed experts as
    lists of (gate, up, down). Offers the accessor methods both the oracle and the GPU
    binding's packer read from."""

    def __init__(self, wl=None, shape=None):
        self.shape = wl.shape if wl is not None else shape
        self.mats = {}
        self.experts = []
        self.shared_mats = []
        self.bias = None
        self.gamma = None
        self.loras = []
        if wl is not None:
            s = wl.shape
            if s.latent_moe:
                self.mats["w_down"] = wl.w_down()
                self.mats["w_up"] = wl.w_up()
            self.mats["w_router"] = wl.w_router()
            g, u, d = wl.routed(0, s.E)
            self.experts = [((g[0][e], g[1][e]), (u[0][e], u[1][e]), (d[0][e], d[1][e])) for e in range(s.E)]
            self.shared_mats = [wl.shared(j) for j in range(s.Ns)]
            self.bias = wl.router_bias()
            self.gamma = wl.rms_gamma()
            if s.lora_rank:
                stack = wl.lora(0, s.E)
                self.loras = [{n: v[e] for n, v in stack.items()} for e in range(s.E)]

    def copy(self):
        return copy.deepcopy(self)

    # accessors
    def w_router(self):
        return self.mats["w_router"]

    def w_down(self):
        return self.mats["w_down"]

    def w_up(self):
        return self.mats["w_up"]

    def routed(self, e, count=1):
        assert count == 1
        return self.experts[e]

    def lora(self, e):
        return self.loras[e]

    def shared(self, j):
        return self.shared_mats[j]

    def router_bias(self):
        return self.bias

    def rms_gamma(self):
        return self.gamma


def identity_mxfp4(n: int):
    """Exact MXFP4 identity [n, n]: one 1.0 per row (code 6 = 4.0 at scale 2^-2)."""
    codes = np.zeros((n, n), np.uint8)
    scales = np.zeros((n, n // 32), np.uint8)
    for i in range(n):
        codes[i, i] = 6
        scales[i, i // 32] = 127 - 2
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def zero_mxfp4(N: int, K: int):
    return np.zeros((N, K // 2), np.uint8), np.zeros((N, K // 32), np.uint8)

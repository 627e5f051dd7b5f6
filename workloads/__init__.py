"""Seeded synthetic workloads for the Kimi K3 LatentMoE layer.

Test and benchmark infrastructure, shared by the CPU oracle and the GPU path:
it draws the token batch and the weights (and the skewed router bias of the
load-imbalance workload) and holds none of the layer's arithmetic.

Shapes follow the Kimi K3 course, lesson 6 "LatentMoE": model width d = 7168,
latent width l = 3584, routed expert GLU hidden 3072, 896 routed experts with
top-16 selection and two full-width shared experts (sections "Deriving the
headline number" and "show me the actual equation"). Weights are drawn
~N(0, 1/fan_in) in fp32 and stored as MXFP4 (E2M1 codes, one E8M0 scale per
32 values along the reduction axis); x ~ N(0, 1) rounded to bf16.

Tensor layout handed to both sides ("canonical MX"):
  codes  uint8 [N, K/2]   element 2i in the low nibble
  scales uint8 [N, K/32]  E8M0 byte
for a matrix W[N, K] that maps K inputs to N outputs (y = W x).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3gen.c")
_LIB = os.path.join(_HERE, "libk3gen.so")

# tensor ids of the counter-based streams
X, W_ROUTER, W_DOWN, W_UP, GATE, UP, DOWN, SH_GATE, SH_UP, SH_DOWN, ZIPF_PERM = range(1, 12)
LORA_A_GATE, LORA_B_GATE, LORA_A_UP, LORA_B_UP, LORA_A_DOWN, LORA_B_DOWN = range(12, 18)
LORA_NAMES = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP). Returns the library path."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


@lru_cache(maxsize=1)
def _lib():
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    u64, u32, i64, i32, f32, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_float, ctypes.c_void_p)
    lib.k3gen_key.argtypes = [u64, u32, u32]
    lib.k3gen_key.restype = u64
    lib.k3gen_u64.argtypes = [u64, u32, u32, i64, vp]
    lib.k3gen_normal.argtypes = [u64, u32, u32, i64, f32, vp]
    lib.k3gen_bf16.argtypes = [u64, u32, u32, i64, f32, vp]
    lib.k3gen_mxfp4_many.argtypes = [u64, u32, u32, i32, i64, i64, f32, vp, vp]
    for f in (lib.k3gen_u64, lib.k3gen_normal, lib.k3gen_bf16, lib.k3gen_mxfp4_many):
        f.restype = None
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def u64(seed: int, tensor: int, sub: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _lib().k3gen_u64(seed, tensor, sub, n, _ptr(out))
    return out


def normal(seed: int, tensor: int, sub: int, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    assert n % 2 == 0
    out = np.empty(n, np.float32)
    _lib().k3gen_normal(seed, tensor, sub, n, std, _ptr(out))
    return out.reshape(shape)


def bf16_normal(seed: int, tensor: int, sub: int, shape, std: float = 1.0) -> np.ndarray:
    """Normals rounded to bf16, returned as raw uint16 bit patterns."""
    n = int(np.prod(shape))
    assert n % 2 == 0
    out = np.empty(n, np.uint16)
    _lib().k3gen_bf16(seed, tensor, sub, n, std, _ptr(out))
    return out.reshape(shape)


def mxfp4(seed: int, tensor: int, sub0: int, N: int, K: int, std: float, count: int | None = None):
    """MXFP4 matrices [N, K] ~ N(0, std^2); with `count`, a stack of `count` of them
    from subs sub0..sub0+count-1. Returns (codes, scales)."""
    assert K % 32 == 0
    c = 1 if count is None else count
    codes = np.empty((c, N, K // 2), np.uint8)
    scales = np.empty((c, N, K // 32), np.uint8)
    _lib().k3gen_mxfp4_many(seed, tensor, sub0, c, N, K, std, _ptr(codes), _ptr(scales))
    if count is None:
        return codes[0], scales[0]
    return codes, scales


# --------------------------------------------------------------------------------------------
# Workload registry
# --------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerShape:
    d: int          # model width
    l: int          # latent width (== d when latent_moe is 0)
    h: int          # routed expert GLU hidden
    E: int          # routed experts
    k: int          # experts selected per token
    Ns: int         # shared experts
    hs: int         # shared expert GLU hidden
    latent_moe: int = 1   # 1: eq. 11 LatentMoE; 0: conventional full-width MoE
    act: str = "bf16"     # activation format of the routed GEMM inputs: "bf16" | "mxfp8"
    eps: float = 1e-6
    lora_rank: int = 0    # rank of the BF16 LoRA deltas on every routed expert matrix (0: none)

    @property
    def expert_in(self) -> int:
        """Width the routed experts work in."""
        return self.l if self.latent_moe else self.d


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    T: int
    seed: int
    bias: str = "zero"        # "zero" | "zipf"
    zipf_alpha: float = 1.5   # b_e = alpha * ln(w_e), w_e Zipf(s=1) weight of expert e's rank
    lora_b_gain: float = 0.25  # standard deviation of a LoRA delta next to the base product (~1)
    note: str = ""

    # ---- inputs -----------------------------------------------------------------------------
    def x_bits(self, T: int | None = None) -> np.ndarray:
        """x [T, d] bf16 bits; rows are the first T rows of the full batch."""
        T = self.T if T is None else T
        return bf16_normal(self.seed, X, 0, (T, self.shape.d))

    def router_bias(self) -> np.ndarray:
        s = self.shape
        if self.bias == "zero":
            return np.zeros(s.E, np.float32)
        # random expert order from the stream; expert at rank r gets Zipf weight 1/(r+1)
        order = np.argsort(u64(self.seed, ZIPF_PERM, 0, s.E), kind="stable")
        rank = np.empty(s.E, np.int64)
        rank[order] = np.arange(s.E)
        w = 1.0 / (rank + 1.0)
        return (self.zipf_alpha * np.log(w)).astype(np.float32)

    def rms_gamma(self) -> np.ndarray:
        return np.ones(self.shape.l, np.float32)

    # ---- weights (canonical MX); std = 1/sqrt(fan_in) -----------------------------------------
    def w_router(self):
        s = self.shape
        return mxfp4(self.seed, W_ROUTER, 0, s.E, s.d, s.d ** -0.5)

    def w_down(self):
        s = self.shape
        return mxfp4(self.seed, W_DOWN, 0, s.l, s.d, s.d ** -0.5)

    def w_up(self):
        s = self.shape
        return mxfp4(self.seed, W_UP, 0, s.d, s.l, s.l ** -0.5)

    def routed(self, e0: int, count: int = 1):
        """Experts e0..e0+count-1: (gate, up, down), each (codes[count,...], scales[count,...]).
        gate/up [h, l'], down [l', h] with l' the expert width."""
        s = self.shape
        li = s.expert_in
        g = mxfp4(self.seed, GATE, e0, s.h, li, li ** -0.5, count=count)
        u = mxfp4(self.seed, UP, e0, s.h, li, li ** -0.5, count=count)
        dn = mxfp4(self.seed, DOWN, e0, li, s.h, s.h ** -0.5, count=count)
        return g, u, dn

    def lora(self, e0: int, count: int | None = None):
        """BF16 LoRA factors of routed expert e0 (or a stack of `count` experts from e0) as bf16 bit
        patterns: a_gate, a_up [r, l'] ~ N(0, 1/l'); a_down [r, h] ~ N(0, 1/h); b_gate, b_up [h, r] and
        b_down [l', r] ~ N(0, (lora_b_gain^2) / r). With v ~ N(0, 1) entries, A v has unit-variance
        entries and the delta B (A v) has standard deviation lora_b_gain (0.25) next to the base
        product's ~1."""
        s = self.shape
        r, li = s.lora_rank, s.expert_in
        assert r > 0
        shapes = {"a_gate": (r, li), "b_gate": (s.h, r), "a_up": (r, li), "b_up": (s.h, r),
                  "a_down": (r, s.h), "b_down": (li, r)}
        stds = {"a_gate": li ** -0.5, "a_up": li ** -0.5, "a_down": s.h ** -0.5,
                "b_gate": self.lora_b_gain * r ** -0.5, "b_up": self.lora_b_gain * r ** -0.5,
                "b_down": self.lora_b_gain * r ** -0.5}
        ids = dict(zip(LORA_NAMES, (LORA_A_GATE, LORA_B_GATE, LORA_A_UP, LORA_B_UP, LORA_A_DOWN, LORA_B_DOWN)))
        c = 1 if count is None else count
        out = {n: np.stack([bf16_normal(self.seed, ids[n], e, shapes[n], stds[n]) for e in range(e0, e0 + c)])
               for n in LORA_NAMES}
        if count is None:
            out = {n: v[0] for n, v in out.items()}
        return out

    def shared(self, j: int):
        s = self.shape
        g = mxfp4(self.seed, SH_GATE, j, s.hs, s.d, s.d ** -0.5)
        u = mxfp4(self.seed, SH_UP, j, s.hs, s.d, s.d ** -0.5)
        dn = mxfp4(self.seed, SH_DOWN, j, s.d, s.hs, s.hs ** -0.5)
        return g, u, dn

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T)


K3 = dict(d=7168, l=3584, h=3072, E=896, k=16, Ns=2, hs=3072)

WORKLOADS = {
    "tiny": Workload("tiny", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=1, hs=96), T=64, seed=0,
                     note="tiny LatentMoE layer, CPU seconds"),
    "tiny_mxfp8": Workload("tiny_mxfp8", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=1, hs=96, act="mxfp8"),
                           T=64, seed=0, note="tiny layer, MXFP8 latent and hidden activations"),
    "tiny_mxfp8_many": Workload("tiny_mxfp8_many", LayerShape(d=256, l=128, h=128, E=16, k=4, Ns=1, hs=96,
                                                              act="mxfp8"), T=512, seed=0,
                                note="tiny layer, MXFP8, 128 rows per expert (scaled-MFMA grouped kernel)"),
    "tiny_mxfp8_deep": Workload("tiny_mxfp8_deep", LayerShape(d=256, l=640, h=768, E=16, k=4, Ns=1, hs=64,
                                                              act="mxfp8"), T=1024, seed=7, bias="zipf",
                                zipf_alpha=0.2,
                                note="tiny layer, MXFP8, several K windows, skewed rows per expert (some above "
                                     "256: several row chunks)"),
    "tiny_bf16_many": Workload("tiny_bf16_many", LayerShape(d=256, l=128, h=128, E=16, k=4, Ns=1, hs=96), T=512,
                               seed=0, note="tiny layer, bf16, 128 rows per expert (row-tiled grouped bf16 kernel)"),
    "tiny_bf16_deep": Workload("tiny_bf16_deep", LayerShape(d=256, l=640, h=768, E=16, k=4, Ns=1, hs=64), T=1024,
                               seed=7, bias="zipf", zipf_alpha=0.2,
                               note="tiny layer, bf16, several K windows, skewed rows per expert (several "
                                    "128-row chunks)"),
    "tiny_split": Workload("tiny_split", LayerShape(d=256, l=128, h=128, E=16, k=2, Ns=1, hs=96), T=128, seed=9,
                           bias="zipf", zipf_alpha=0.3,
                           note="tiny layer, bf16, 16 rows per expert on average with a skewed load: experts "
                                "of 32 or more rows on the row-tiled kernel, the others on the panel kernel"),
    "tiny_split_mxfp8": Workload("tiny_split_mxfp8", LayerShape(d=256, l=128, h=128, E=16, k=2, Ns=1, hs=96,
                                                                act="mxfp8"), T=128, seed=9, bias="zipf",
                                 zipf_alpha=0.3, note="as tiny_split with MXFP8 latent and hidden activations"),
    "tiny_e12_mxfp8": Workload("tiny_e12_mxfp8", LayerShape(d=256, l=128, h=128, E=12, k=3, Ns=1, hs=96,
                                                            act="mxfp8"), T=512, seed=10,
                               note="tiny layer, MXFP8, 12 experts (XCD classes of unequal size), many rows"),
    "tiny_e4_bf16": Workload("tiny_e4_bf16", LayerShape(d=256, l=128, h=128, E=4, k=2, Ns=1, hs=96), T=256,
                             seed=11, note="tiny layer, bf16, 4 experts (XCD classes without experts), many rows"),
    "tiny_e4_all": Workload("tiny_e4_all", LayerShape(d=256, l=128, h=96, E=4, k=4, Ns=1, hs=96), T=128, seed=17,
                            note="tiny layer, bf16, 4 experts each chosen by every token: the batch size sets every "
                                 "expert's row count exactly (kernel band boundaries), K tail in the down GEMM"),
    "tiny_e4_all_mxfp8": Workload("tiny_e4_all_mxfp8", LayerShape(d=256, l=128, h=128, E=4, k=4, Ns=1, hs=96,
                                                                  act="mxfp8"), T=128, seed=18,
                                  note="as tiny_e4_all with MXFP8 latent and hidden activations"),
    "tiny_dense_many": Workload("tiny_dense_many", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=1, hs=96), T=2048,
                                seed=8, note="tiny layer, bf16, 2048 tokens (row-tiled dense GEMMs, K tail "
                                             "in the latent/shared GEMM)"),
    "tiny_fullwidth": Workload("tiny_fullwidth", LayerShape(d=256, l=256, h=96, E=16, k=2, Ns=1, hs=96,
                                                            latent_moe=0), T=64, seed=5,
                               note="tiny conventional full-width MoE"),
    "tiny_skewed": Workload("tiny_skewed", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=2, hs=64), T=96,
                            seed=6, bias="zipf", zipf_alpha=0.3, note="tiny layer, Zipf-skewed bias, two shared"),
    "tiny_lora": Workload("tiny_lora", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=1, hs=96, lora_rank=16), T=64,
                          seed=12, note="tiny layer, rank-16 BF16 LoRA deltas on every routed expert matrix (panel "
                                        "kernels)"),
    "tiny_lora_mxfp8_many": Workload("tiny_lora_mxfp8_many", LayerShape(d=256, l=256, h=128, E=16, k=4, Ns=1, hs=96,
                                                                        act="mxfp8", lora_rank=8), T=512, seed=13,
                                     note="tiny layer, MXFP8, rank-8 LoRA, 128 rows per expert (scaled-MFMA "
                                          "row-tiled kernels)"),
    "tiny_lora_bf16_many": Workload("tiny_lora_bf16_many", LayerShape(d=256, l=128, h=128, E=16, k=4, Ns=1, hs=96,
                                                                      lora_rank=32), T=512, seed=14,
                                    note="tiny layer, bf16, rank-32 LoRA, 128 rows per expert (bf16 row-tiled "
                                         "kernels)"),
    "tiny_lora_r32_skewed": Workload("tiny_lora_r32_skewed", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=1, hs=96,
                                                                        lora_rank=32), T=31, seed=15, bias="zipf",
                                     zipf_alpha=1.5,
                                     note="tiny layer, rank-32 LoRA, literal Zipf bias: hot experts of more than 16 "
                                          "rows on the panel kernel (two row tiles)"),
    "tiny_lora_mxfp8_r8": Workload("tiny_lora_mxfp8_r8", LayerShape(d=256, l=128, h=96, E=16, k=4, Ns=1, hs=96,
                                                                    act="mxfp8", lora_rank=8), T=40, seed=16,
                                   note="tiny layer, MXFP8, rank-8 LoRA, 10 rows per expert (panel and row-tiled "
                                        "kernels in one stage)"),
    "tiny_lora_split": Workload("tiny_lora_split", LayerShape(d=256, l=128, h=128, E=16, k=2, Ns=1, hs=96,
                                                              lora_rank=16), T=128, seed=9, bias="zipf",
                                zipf_alpha=0.3,
                                note="as tiny_split with rank-16 LoRA: panel and row-tiled kernels in one stage"),
    "k3_decode_t64": Workload("k3_decode_t64", LayerShape(**K3), T=64, seed=1,
                              note="K3 shape decode, uniform routing (b = 0)"),
    "k3_decode_t512_zipf": Workload("k3_decode_t512_zipf", LayerShape(**K3), T=512, seed=1, bias="zipf",
                                    zipf_alpha=1.5,
                                    note="K3 shape decode, literal Zipf bias b = 1.5 ln w"),
    "k3_decode_t512_zipf_cal": Workload("k3_decode_t512_zipf_cal", LayerShape(**K3), T=512, seed=1,
                                        bias="zipf", zipf_alpha=0.03,
                                        note="K3 shape decode, Zipf bias scaled to a 2-10x hot-expert load"),
    "k3_prefill_t8192": Workload("k3_prefill_t8192", LayerShape(**K3, act="mxfp8"), T=8192, seed=3,
                                 note="K3 shape prefill chunk, MXFP8 latent and hidden activations"),
    "k3_decode_t64_lora": Workload("k3_decode_t64_lora", LayerShape(**K3, lora_rank=16), T=64, seed=1,
                                   note="K3 shape decode (the T = 64 batch and weights of k3_decode_t64) with "
                                        "rank-16 BF16 LoRA deltas on every routed expert matrix"),
    "k3_t2048": Workload("k3_t2048", LayerShape(**K3), T=2048, seed=3,
                         note="K3 shape, 2048 tokens, bf16 activations (the LatentMoE side of the "
                              "full-width T = 2048 comparison)"),
    "fullwidth_t64": Workload("fullwidth_t64", LayerShape(d=7168, l=7168, h=3072, E=896, k=8, Ns=2, hs=3072,
                                                          latent_moe=0), T=64, seed=4,
                              note="conventional full-width MoE, top-8"),
    "fullwidth_t2048": Workload("fullwidth_t2048", LayerShape(d=7168, l=7168, h=3072, E=896, k=8, Ns=2,
                                                              hs=3072, latent_moe=0), T=2048, seed=4,
                                note="conventional full-width MoE, top-8"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def fingerprint(wl: Workload) -> dict:
    """sha256 of a workload's canonical inputs (bf16 bit patterns, MX codes and scales as stored): the
    whole x batch, the router bias, the dense matrices, every shared expert, the first and last routed
    expert (and their LoRA factors). A change of the generator or of a seed shows here."""
    import hashlib
    s = wl.shape

    def h(*arrays):
        d = hashlib.sha256()
        for a in arrays:
            a = np.ascontiguousarray(a)
            d.update(str((a.dtype.str, a.shape)).encode())
            d.update(a.tobytes())
        return d.hexdigest()

    out = {"x": h(wl.x_bits()), "router_bias": h(wl.router_bias()), "w_router": h(*wl.w_router())}
    if s.latent_moe:
        out["w_down"] = h(*wl.w_down())
        out["w_up"] = h(*wl.w_up())
    for j in range(s.Ns):
        out[f"shared{j}"] = h(*(a for m in wl.shared(j) for a in m))
    for e in sorted({0, s.E - 1}):
        out[f"expert{e}"] = h(*(a for m in wl.routed(e) for a in m))
        if s.lora_rank:
            lo = wl.lora(e)
            out[f"lora{e}"] = h(*(lo[n] for n in LORA_NAMES))
    return out

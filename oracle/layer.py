"""fp64 definition of the Kimi K3 LatentMoE layer forward.

TEST INFRASTRUCTURE (see the package docstring).

Source: Kimi K3 course, lesson 6 "LatentMoE", section "show me the actual
equation":

  eq. 11   u = sum_{i in T_k(x)} p_i * E_i^routed(W_down x)          (in R^l)
           y = sum_{j=1..N_s} E_j^shared(x) + W_up RMSNorm(u)        (in R^d)
  eq. 13   s = Sigmoid(W_r x);  T = argtopk(s + b);  p_j = s_j / sum_{r in T} s_r

with routed experts mapping R^l -> R^l, shared experts R^d -> R^d, the bias b
steering selection only, and the RMSNorm applied to the aggregated routed
output before the up-projection (section "What extreme sparsity breaks").
The conventional full-width MoE the lesson compares against ("The problem with
a big expert pool", table "What scales with what") drops W_down, W_up and the
RMSNorm: y = sum shared + sum p_i E_i(x) with experts at width d.

Readings where the pages leave a step open (each also listed in the design notes):
* Expert network: a SwiGLU GLU, h = SiLU(W_gate z) * (W_up_e z), o = W_down_e h
  (each routed expert is a GLU with gate, up and down matrices; lesson 6, "Deriving the
  headline number").
* Router input is the full-width x (eq. 13 writes W_r x).
* Top-k order: descending key, equal keys -> lower expert id first.
* RMSNorm: n = gamma * u / sqrt(mean(u^2) + eps).
* Shared experts take the raw x and are the same GLU at width d.
* BF16 LoRA deltas ("Serving K3, 01 architecture", the paragraph on the MXFP4 KL floor: fine-tuning
  ships BF16 LoRA deltas over the MXFP4 base weights): when the shape has lora_rank r > 0, every
  routed expert matrix W [N, K] (gate, up, down) is W + B A with bf16 A [r, K] and B [N, r]; the
  product is exact in fp64, so the delta is taken as B (A v) on the activation v the base matrix
  sees. Shared experts and the dense projections carry no deltas.
* Quantisation points (the workload's definition): x arrives as bf16; the
  latent z fed to the experts and the GLU hidden h are rounded to bf16
  ("bf16" workloads) or MX-encoded as MXFP8 in blocks of 32 along the feature
  axis ("mxfp8" workloads); n and the shared hidden are rounded to bf16; expert
  outputs, u and y stay fp64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import mx


# ----------------------------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------------------------

def sigmoid(a):
    """Logistic function 1 / (1 + e^-a) (eq. 13)."""
    return 1.0 / (1.0 + np.exp(-a))


def silu(g):
    """SiLU(g) = g * sigmoid(g), the gate nonlinearity of a SwiGLU GLU."""
    return g / (1.0 + np.exp(-g))


def q_act(v, act: str):
    """Quantisation point of a routed-path activation.
    Returns (fp64 values after quantisation, codes or None, scale bytes or None)."""
    if act == "bf16":
        q = mx.bf16_round(v)
        return q, None, None
    if act == "mxfp8":
        codes, scales = mx.mx_quantize(v, "e4m3")
        return mx.mx_dequantize(codes, scales, "e4m3"), codes, scales
    raise ValueError(act)


def rmsnorm(u, gamma, eps):
    """n = gamma * u / sqrt(mean(u^2) + eps), over the last axis (lesson 6, RMSNorm before W_up)."""
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return np.asarray(gamma, np.float64) * u / np.sqrt(ms + eps)


# ----------------------------------------------------------------------------------------------
# router (eq. 13)
# ----------------------------------------------------------------------------------------------

def router_scores(xh, Wr):
    """s = Sigmoid(W_r x) for every token: [T, d] x [E, d] -> [T, E]."""
    return sigmoid(xh @ Wr.T)


@dataclass
class Selection:
    idx: np.ndarray        # [T, k] selected experts, in rank order
    key_sorted: np.ndarray  # [T, k+1] the k+1 largest keys, descending
    key: np.ndarray        # [T, E] s + b

    def boundary_gap(self):
        """Key gap between ranks k and k+1 (1-based) per token."""
        return self.key_sorted[:, -2] - self.key_sorted[:, -1]

    def adjacent_gaps(self):
        return self.key_sorted[:, :-2] - self.key_sorted[:, 1:-1]


def select_topk(s, b, k: int) -> Selection:
    """T = argtopk(s + b): the k largest keys, descending; equal keys -> lower id first."""
    key = s + np.asarray(b, np.float64)[None, :]
    T, E = key.shape
    ids = np.broadcast_to(np.arange(E), key.shape)
    order = np.lexsort((ids, -key), axis=-1)          # primary -key, secondary id
    take = min(k + 1, E)
    sel = order[:, :take]
    ks = np.take_along_axis(key, sel, axis=1)
    if take == k:                                     # k == E: no rank k+1
        ks = np.concatenate([ks, np.full((T, 1), -np.inf)], axis=1)
    return Selection(idx=sel[:, :k].astype(np.int64), key_sorted=ks, key=key)


def renorm(s, idx):
    """p_j = s_j / sum_{r in T} s_r, from the unbiased scores (eq. 13)."""
    ss = np.take_along_axis(s, idx, axis=1)
    return ss / ss.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------------------------
# dispatch: expert-contiguous rows
# ----------------------------------------------------------------------------------------------

def routing_tables(idx, E: int):
    """Rows of the dispatched batch, ordered by (expert ascending, token ascending).
    counts[e] = #(t, j) with idx[t, j] = e; offsets = exclusive prefix sum (length E+1);
    perm[row] = token of that row; inv[t, j] = row of (t, j)."""
    T, k = idx.shape
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    counts = np.bincount(flat_e, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.lexsort((flat_t, flat_e))              # primary expert, secondary token
    perm = flat_t[order]
    inv = np.empty(T * k, np.int64)
    inv[order] = np.arange(T * k)
    return counts, offsets, perm, inv.reshape(T, k)


# ----------------------------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------------------------

def with_delta(v, W, ab=None):
    """v W^T, plus the LoRA delta (v A^T) B^T when ab = (A, B) is given: v (W + B A)^T."""
    out = v @ W.T
    if ab is not None:
        A, B = ab
        out = out + (v @ A.T) @ B.T
    return out


def glu(zq, G, U, D, act: str, lora=None):
    """One GLU expert on a batch of rows: h = Q(SiLU(zq G^T) * (zq U^T)), o = h D^T, each matrix with
    its LoRA delta when `lora` (dict of fp64 factors a_gate, b_gate, a_up, b_up, a_down, b_down) is given.
    Returns (o, hq, h pre-quantisation, h codes, h scales)."""
    lg = (lora["a_gate"], lora["b_gate"]) if lora else None
    lu = (lora["a_up"], lora["b_up"]) if lora else None
    ld = (lora["a_down"], lora["b_down"]) if lora else None
    g = with_delta(zq, G, lg)
    v = with_delta(zq, U, lu)
    hpre = silu(g) * v
    hq, hc, hs = q_act(hpre, act)
    return with_delta(hq, D, ld), hq, hpre, hc, hs


def lora_factors(weights, e, shape):
    """fp64 LoRA factors of routed expert e (bf16 values, exact), or None without deltas."""
    if not getattr(shape, "lora_rank", 0):
        return None
    return {k: mx.bf16_from_bits(v) for k, v in weights.lora(e).items()}


def dequant(mxpair):
    codes, scales = mxpair
    return mx.mxfp4_matrix(codes, scales)


@dataclass
class Result:
    y: np.ndarray
    taps: dict = field(default_factory=dict)


def forward(x_bits, weights, shape, select_override=None, keep_expert_rows=True, z_override=None,
            h_override=None) -> Result:
    """The layer on a batch of tokens.

    x_bits: bf16 bit patterns [T, d]. weights: object with w_router(), w_down(), w_up(),
    routed(e) -> (gate, up, down), shared(j) -> (gate, up, down), router_bias(), rms_gamma(),
    matrices as canonical MXFP4 (codes [N, K/2], scales [N, K/32]).
    select_override: optional {token index: sequence of k expert ids} used instead of
    the oracle's own top-k for those tokens (to score a GPU selection that differs
    only inside the tie tolerance).
    z_override [T, l] / h_override [T, k, h]: optional values after the quantisation point
    of the latent z / the GLU hidden of (token, selection slot), used instead of the
    oracle's own quantisation, so that a quantisation decision is taken on the value the
    compared implementation computed (its codes are checked against this oracle's encoder
    separately).
    """
    s_ = shape
    xh = mx.bf16_from_bits(x_bits)
    T = xh.shape[0]
    taps = {}

    # router, eq. 13
    Wr = dequant(weights.w_router())
    s = router_scores(xh, Wr)
    sel = select_topk(s, weights.router_bias(), s_.k)
    idx = sel.idx.copy()
    if select_override:
        for t, ids in select_override.items():
            idx[t] = np.asarray(ids, np.int64)
    p = renorm(s, idx)
    taps.update(scores=s, selection=sel, idx=idx, p=p)

    # routed input: W_down x then the quantisation point (latent), or x itself (full width)
    if s_.latent_moe:
        z = xh @ dequant(weights.w_down()).T
        zq, zc, zs = q_act(z, s_.act)
        if z_override is not None:
            zq = np.asarray(z_override, np.float64)
        taps.update(z=z, zq=zq, z_codes=zc, z_scales=zs)
    else:
        zq = xh

    counts, offsets, perm, inv = routing_tables(idx, s_.E)
    taps.update(counts=counts, offsets=offsets, perm=perm, inv=inv)

    # routed experts, one expert at a time over its dispatched rows (expert-contiguous order)
    width = s_.expert_in
    rows_out = np.zeros((T * s_.k, width))
    rows_h = np.zeros((T * s_.k, s_.h)) if keep_expert_rows else None
    rows_hpre = np.zeros((T * s_.k, s_.h)) if keep_expert_rows else None
    row_tj = np.empty((T * s_.k, 2), np.int64)          # dispatched row -> (token, slot)
    row_tj[inv.reshape(-1)] = np.stack(np.meshgrid(np.arange(T), np.arange(s_.k), indexing="ij"), -1).reshape(-1, 2)
    for e in np.nonzero(counts)[0]:
        r0, r1 = offsets[e], offsets[e + 1]
        (gc, uc, dc) = weights.routed(int(e))
        G, U, D = dequant(_first(gc)), dequant(_first(uc)), dequant(_first(dc))
        lo = lora_factors(weights, int(e), s_)
        o, hq, hpre, _, _ = glu(zq[perm[r0:r1]], G, U, D, s_.act, lo)
        if h_override is not None:
            hq = np.asarray(h_override, np.float64)[row_tj[r0:r1, 0], row_tj[r0:r1, 1]]
            o = with_delta(hq, D, (lo["a_down"], lo["b_down"]) if lo else None)
        rows_out[r0:r1] = o
        if keep_expert_rows:
            rows_h[r0:r1] = hq
            rows_hpre[r0:r1] = hpre
    taps.update(expert_out=rows_out, h=rows_h, hpre=rows_hpre)

    # p-weighted combine in selection order, eq. 11
    o_tk = rows_out[inv]                               # [T, k, width]
    u = np.einsum("tk,tkc->tc", p, o_tk)
    taps["u"] = u

    if s_.latent_moe:
        npre = rmsnorm(u, weights.rms_gamma(), s_.eps)
        n = mx.bf16_round(npre)
        y_routed = n @ dequant(weights.w_up()).T
        taps.update(n=n, n_pre=npre)
    else:
        y_routed = u

    # shared experts on the raw x, full width
    y_shared = np.zeros((T, s_.d))
    hs_list = []
    for j in range(s_.Ns):
        gc, uc, dc = weights.shared(j)
        o, hq, _, _, _ = glu(xh, dequant(gc), dequant(uc), dequant(dc), "bf16")
        y_shared += o
        hs_list.append(hq)
    taps.update(y_shared=y_shared, hs=hs_list, y_routed=y_routed)

    return Result(y=y_shared + y_routed, taps=taps)


# ----------------------------------------------------------------------------------------------
# expert-parallel send side ("Serving K3, 01 architecture": experts sharded over accelerators, an
# all-to-all of data-dependent sizes; "Kimi K3: architectural innovations", "Compress the expert
# interface": what crosses is the latent). Experts in n_ranks contiguous ranges of E / n_ranks.
# ----------------------------------------------------------------------------------------------

def ep_send_counts(idx, E: int, n_ranks: int):
    """Rows each rank receives: the number of (token, slot) pairs whose expert lies in its range."""
    assert E % n_ranks == 0
    per = E // n_ranks
    dest = np.asarray(idx, np.int64).reshape(-1) // per
    return np.bincount(dest, minlength=n_ranks).astype(np.int64)


def ep_send_rows(routed_in, perm):
    """The send buffer: the routed input (z after its quantisation point, or x at full width) of every
    dispatched row, in dispatched order (expert ascending, token ascending) -- grouped by destination."""
    return np.asarray(routed_in)[np.asarray(perm, np.int64)]


def _first(pair):
    """Accept either a single matrix (codes, scales) or a stack of one."""
    c, sc = pair
    if c.ndim == 3:
        return c[0], sc[0]
    return c, sc


def check_selection(gpu_idx, sel: Selection, tol: float = 1e-6):
    """Compare a GPU top-k against the oracle's.

    A token's GPU list is accepted when it holds k distinct experts and its j-th
    pick has an oracle key within `tol` of the oracle's j-th largest key for every
    j (so it differs only where keys tie to within `tol`). Returns
    (ok mask [T], flip mask [T]): flip = accepted but not identical."""
    gpu_idx = np.asarray(gpu_idx, np.int64)
    T, k = gpu_idx.shape
    distinct = np.array([len(set(r.tolist())) == k for r in gpu_idx])
    in_range = (gpu_idx >= 0) & (gpu_idx < sel.key.shape[1])
    safe = np.where(in_range, gpu_idx, 0)
    kg = np.take_along_axis(sel.key, safe, axis=1)
    close = np.abs(kg - sel.key_sorted[:, :k]) < tol
    ok = distinct & in_range.all(axis=1) & close.all(axis=1)
    same = (gpu_idx == sel.idx).all(axis=1)
    return ok, ok & ~same

"""Comparison helpers for GPU-vs-oracle parity (tolerances stated where they are used)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import layer, mx

# Output bar: relative L2 <= 5e-3 and max-abs <= 2e-2 * rms(y_oracle).
Y_REL_L2 = 5e-3
Y_MAXABS_RMS = 2e-2
# Selection flips are allowed where oracle keys tie to within this (fp64) gap.
KEY_TIE = 1e-6


def np64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def y_metrics(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    rel = np.linalg.norm(y_gpu - y_ref) / np.linalg.norm(y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2))
    maxabs = np.max(np.abs(y_gpu - y_ref))
    return rel, maxabs / rms


def assert_y(y_gpu, y_ref, what="y"):
    rel, ma = y_metrics(y_gpu, y_ref)
    assert rel <= Y_REL_L2, f"{what}: relative L2 {rel:.3g} > {Y_REL_L2}"
    assert ma <= Y_MAXABS_RMS, f"{what}: max-abs {ma:.3g} * rms > {Y_MAXABS_RMS}"
    return rel, ma


U32 = 2.0 ** -24


def dot_error_bound(abs_a, abs_w):
    """Bound on |fp32 accumulation - exact| for rows of A times rows of W: 8 sqrt(K) u sum|a||w|
    (u = 2^-24; the sqrt(K) growth of rounding errors of a K-term sum with a safety factor 8)."""
    K = abs_a.shape[-1]
    return 8.0 * np.sqrt(K) * U32 * (abs_a @ abs_w.T) + 1e-30


def check_bf16_quant(gpu_bits, gpu_pre, oracle_pre, bound):
    """bf16 quantisation point. Strict: the oracle's rounding of the GPU's own fp32 value gives
    the GPU's bits. Accuracy: |GPU fp32 value - oracle value| <= bound. Rounding is monotone, so
    a GPU value then differs from bf16(oracle value) only where a rounding boundary lies between
    the two. Returns the number of such differences."""
    got = mx.bf16_from_bits(gpu_bits)
    gpu_pre = np.asarray(gpu_pre, np.float64)
    assert np.array_equal(mx.bf16_round(gpu_pre), got), "GPU bf16 rounding"
    err = np.abs(gpu_pre - oracle_pre)
    assert np.all(err <= bound), f"pre-quantisation value off by {np.max(err / bound):.3g} x the bound"
    return int((got != mx.bf16_round(oracle_pre)).sum())


def check_mx_quant(gpu_codes, gpu_scales, gpu_pre, oracle_pre, bound, fmt="e4m3"):
    """MX quantisation point (bit-exact codes). Strict: the oracle's MX encoder on the GPU's own
    fp32 values reproduces the GPU's codes and scales. Accuracy: |GPU fp32 value - oracle value|
    <= bound. Returns the number of codes that differ from the oracle's encoding of its own values
    (each one a block amax or element on the other side of a boundary within the bound)."""
    gpu_pre = np.asarray(gpu_pre, np.float64)
    c2, s2 = mx.mx_quantize(gpu_pre, fmt)
    assert np.array_equal(c2, gpu_codes), "GPU MX codes differ from the oracle encoding of the GPU's values"
    assert np.array_equal(s2, gpu_scales), "GPU MX scales differ from the oracle encoding of the GPU's values"
    err = np.abs(gpu_pre - oracle_pre)
    assert np.all(err <= bound), f"pre-quantisation value off by {np.max(err / bound):.3g} x the bound"
    c3, s3 = mx.mx_quantize(oracle_pre, fmt)
    return int(((c3 != gpu_codes) | np.repeat(s3 != gpu_scales, 32, axis=-1)).sum())


# The scaled MFMA (MXFP8 x MXFP4, 128-wide K windows) accumulates each window's products with an error
# measured at about 2^-16 of the window's sum of magnitudes (reading R26); doubled, and summed over the
# windows, that is 2^-15 of the whole sum of magnitudes.
SCALED_MFMA_REL = 2.0 ** -15


def glu_hidden_bound(zr, G, U, lo=None, scaled_mfma=False):
    """Exact fp64 GLU hidden SiLU(zr G'^T) * (zr U'^T) of some rows (G', U' the matrices with their LoRA
    deltas when `lo` is given) and a bound on an fp32 implementation's error in it: the dot-product
    bound of each product (with the LoRA factor's magnitudes added to the weights', and a second
    accumulation of rank terms; with `scaled_mfma`, plus the scaled MFMA's window term), propagated
    through SiLU (|SiLU'| <= 1.1) and the product, plus 16 fp32 roundings of the result for the
    SiLU's exponential, reciprocal and products."""
    az = np.abs(zr)
    K = zr.shape[1]

    def prod(W, a, b):
        mag = az @ np.abs(W).T
        if lo is None:
            return zr @ W.T, dot_error_bound(az, np.abs(W)) + (SCALED_MFMA_REL * mag if scaled_mfma else 0.0)
        A, B = lo[a], lo[b]
        t = zr @ A.T
        val = zr @ W.T + t @ B.T
        bnd = 8.0 * np.sqrt(K) * U32 * (az @ (np.abs(W) + np.abs(B) @ np.abs(A)).T)
        bnd += 8.0 * np.sqrt(A.shape[0]) * U32 * (np.abs(t) @ np.abs(B).T) + 1e-30
        if scaled_mfma:
            bnd += SCALED_MFMA_REL * mag
        return val, bnd

    g, bg = prod(G, "a_gate", "b_gate")
    v, bv = prod(U, "a_up", "b_up")
    sg = layer.silu(g)
    h = sg * v
    bound = 1.1 * bg * (np.abs(v) + bv) + (np.abs(sg) + 1.1 * bg) * bv + 16.0 * U32 * np.abs(h) + 1e-30
    return h, bound


def check_routing(gpu, sel, E):
    """Selection within key ties, and dispatch tables bit-exact for the GPU's selection."""
    idx = gpu["topk_idx"].astype(np.int64)
    ok, flip = layer.check_selection(idx, sel, tol=KEY_TIE)
    assert ok.all(), f"selection differs beyond key ties for tokens {np.nonzero(~ok)[0][:10]}"
    counts, offsets, perm, inv = layer.routing_tables(idx, E)
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offsets"], offsets)
    assert np.array_equal(gpu["perm"], perm)
    assert np.array_equal(gpu["inv"].reshape(inv.shape), inv)
    return int(flip.sum())


def decode_act(codes_or_bits, scales, act):
    """GPU activation at its quantisation point -> fp64 values (bf16 bits, or E4M3 codes + scales)."""
    if act == "mxfp8":
        return mx.mx_dequantize(codes_or_bits, scales, "e4m3")
    return mx.bf16_from_bits(codes_or_bits)


def stagewise(g, weights, shape, x_bits):
    """Each routed-path kernel against the oracle's definition of its step applied to the GPU's own
    inputs (the quantisation decisions taken in the GPU's precision, pinned separately by the strict
    encoder checks). Returns a dict of relative errors; asserts them."""
    s = shape
    T = x_bits.shape[0]
    act = s.act
    out = {}
    if s.latent_moe:
        zq = decode_act(g["z"], g.get("z_scales"), act)
    else:
        zq = mx.bf16_from_bits(x_bits)
    hq = decode_act(g["h"], g.get("h_scales"), act)
    perm, offsets = g["perm"], g["offsets"]
    h_ref = np.zeros_like(g["h_f32"], dtype=np.float64)
    o_ref = np.zeros_like(g["expert_out"], dtype=np.float64)
    for e in np.nonzero(g["counts"])[0]:
        r0, r1 = offsets[e], offsets[e + 1]
        G, U, D = (layer.dequant(m) for m in _first3(weights.routed(int(e))))
        lo = layer.lora_factors(weights, int(e), s)
        zr = zq[perm[r0:r1]]
        pair = (lambda a, b: (lo[a], lo[b]) if lo else None)  # noqa: E731
        h_ref[r0:r1] = layer.silu(layer.with_delta(zr, G, pair("a_gate", "b_gate"))) * \
            layer.with_delta(zr, U, pair("a_up", "b_up"))
        o_ref[r0:r1] = layer.with_delta(hq[r0:r1], D, pair("a_down", "b_down"))
    out["h"] = rel_l2(g["h_f32"], h_ref)
    out["o"] = rel_l2(g["expert_out"], o_ref)
    inv = g["inv"].reshape(T, s.k)
    u_ref = np.einsum("tk,tkc->tc", g["topk_p"].astype(np.float64), g["expert_out"].astype(np.float64)[inv])
    out["u"] = rel_l2(g["u"], u_ref)
    # 1e-4: the fp8 x fp4 scaled MFMA accumulates with ~2^-16 relative error (measured); logic
    # errors (a wrong row, scale or operand) show up as O(1)
    assert out["h"] < 1e-4 and out["o"] < 1e-4 and out["u"] < 1e-6, out
    if s.latent_moe:
        npre = layer.rmsnorm(g["u"].astype(np.float64), weights.rms_gamma(), s.eps)
        out["n_diff"] = int((mx.bf16_from_bits(g["n"]) != mx.bf16_round(npre)).sum())
        assert out["n_diff"] <= max(2, 1e-3 * npre.size)
        parity_n = rel_l2(mx.bf16_from_bits(g["n"]), npre)
        assert parity_n < 4e-3
    return out


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _first3(m):
    def one(p):
        c, sc = p
        return (c[0], sc[0]) if c.ndim == 3 else (c, sc)
    return tuple(one(p) for p in m)

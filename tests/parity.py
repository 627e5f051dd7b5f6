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
        zr = zq[perm[r0:r1]]
        h_ref[r0:r1] = layer.silu(zr @ G.T) * (zr @ U.T)
        o_ref[r0:r1] = hq[r0:r1] @ D.T
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

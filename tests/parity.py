"""Comparison helpers for GPU-vs-oracle parity (tolerances stated where they are used)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import layer, mx

# Output bar: relative L2 <= 5e-3 and max-abs <= 2e-2 * rms(y_oracle).
Y_REL_L2 = 5e-3
Y_MAXABS_RMS = 2e-2
# A quantisation decision may differ from the oracle's only where the oracle's value (divided by
# its block scale) lies within this relative distance of a rounding midpoint, or the block's amax
# within it of a power of two: fp32 accumulation on the GPU moves values by ~1e-6 relative.
MIDPOINT_BAND = 2.0 ** -16
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


def near_bf16_midpoint(v):
    """True where fp64 v lies within MIDPOINT_BAND (relative) of a bf16 rounding midpoint."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.exp2(e - 7)
    frac = a / q - np.floor(a / q)
    return np.abs(frac - 0.5) * q <= MIDPOINT_BAND * np.maximum(a, 1e-300)


def check_bf16_quant(gpu_bits, gpu_pre, oracle_pre):
    """bf16 quantisation point. Strict: the oracle's rounding of the GPU's own fp32 value gives
    the GPU's bits. End to end: a GPU value differs from bf16(oracle value) only where the oracle
    value sits at a rounding midpoint. Returns the number of such allowed differences."""
    got = mx.bf16_from_bits(gpu_bits)
    assert np.array_equal(mx.bf16_round(np.asarray(gpu_pre, np.float64)), got), "GPU bf16 rounding"
    ref = mx.bf16_round(oracle_pre)
    diff = got != ref
    assert np.all(near_bf16_midpoint(np.asarray(oracle_pre)[diff])), "bf16 value differs away from a midpoint"
    return int(diff.sum())


def near_mx_boundary(v, fmt):
    """Per element: oracle value / X within MIDPOINT_BAND of a rounding midpoint of the element
    grid, or block amax within MIDPOINT_BAND of a power of two."""
    v = np.asarray(v, np.float64)
    codes, sb = mx.mx_quantize(v, fmt)
    X = np.repeat(mx.e8m0_value(sb), 32, axis=-1)
    x = np.abs(v / X)
    table = mx.E2M1_TABLE if fmt == "e2m1" else mx.E4M3_TABLE
    grid = np.unique(np.abs(table[np.isfinite(table)]))
    mids = (grid[:-1] + grid[1:]) / 2
    dist = np.min(np.abs(x[..., None] - mids), axis=-1)
    near_mid = dist <= MIDPOINT_BAND * np.maximum(x, 1e-300)
    K = v.shape[-1]
    amax = np.abs(v.reshape(v.shape[:-1] + (K // 32, 32))).max(axis=-1)
    lg = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = np.abs(lg - np.round(lg)) <= MIDPOINT_BAND * 2
    return near_mid | np.repeat(near_pow2, 32, axis=-1)


def check_mx_quant(gpu_codes, gpu_scales, gpu_pre, oracle_pre, fmt="e4m3"):
    """MX quantisation point (bit-exact codes). Strict: the oracle's MX encoder on the GPU's own
    fp32 values reproduces the GPU's codes and scales. End to end: codes differ from the oracle's
    encoding of its own values only at rounding boundaries. Returns the count of such codes."""
    c2, s2 = mx.mx_quantize(np.asarray(gpu_pre, np.float64), fmt)
    assert np.array_equal(c2, gpu_codes), "GPU MX codes differ from the oracle encoding of the GPU's values"
    assert np.array_equal(s2, gpu_scales), "GPU MX scales differ from the oracle encoding of the GPU's values"
    c3, s3 = mx.mx_quantize(oracle_pre, fmt)
    diff = (c3 != gpu_codes) | np.repeat(s3 != gpu_scales, 32, axis=-1)
    assert np.all(near_mx_boundary(oracle_pre, fmt)[diff]), "MX code differs away from a rounding boundary"
    return int(diff.sum())


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

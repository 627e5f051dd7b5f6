"""Exact fp64 codec for the number formats the layer uses.

TEST INFRASTRUCTURE (see the package docstring).

Formats (OCP Microscaling Formats v1.0, the reading fixed for this repository;
the specification itself is not among the pages, which only say the K3 weights
are MXFP4 and the activations MXFP8 -- serving article, section on quantisation
as a property of the artefact; architectural-innovations article, "Launch-level
facts"):

* E2M1 (FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 (FP8, "fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
  largest finite 448, S.1111.111 is NaN, no inf.
* E8M0 scale: 2^(byte - 127); byte 255 is NaN.
* MX block: 32 consecutive elements share one E8M0 scale X.
  Encoding a block V: if max|V| = 0 the scale byte is 0 and every element is
  zero; otherwise X = 2^e with e = floor(log2 max|V|) - emax_elem (emax_elem = 2
  for E2M1, 8 for E4M3) clamped to [-127, 127], and each element is V_i / X
  rounded to nearest, ties to even, on the element grid, saturating at the
  largest finite magnitude; the sign of a zero result is kept.
* bf16: 8 exponent bits, 7 stored mantissa bits, round to nearest even.

Codes are handled unpacked (one integer per element); `pack_fp4`/`unpack_fp4`
convert to the two-per-byte exchange layout (element 2i in the low nibble).
"""
from __future__ import annotations

import numpy as np

# (mantissa bits, minimum normal exponent, largest finite magnitude, emax of the element format)
FORMATS = {
    "e2m1": (1, 0, 6.0, 2),
    "e4m3": (3, -6, 448.0, 8),
}


def e2m1_value(code: int) -> float:
    """Decode one E2M1 code (0..15) from its bit fields."""
    sign = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m                      # subnormal: 2^(1-1) * m/2
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


def e4m3_value(code: int) -> float:
    """Decode one E4M3 ("fn") code (0..255) from its bit fields."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = 2.0 ** -6 * (m / 8.0)         # subnormal
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], np.float64)


def e8m0_value(byte):
    b = np.asarray(byte, np.float64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def round_to_grid(v, mbits: int, emin: int, maxval: float | None):
    """Round fp64 values to nearest-even on a binary floating-point grid with `mbits`
    stored mantissa bits and smallest normal exponent `emin` (subnormals kept).
    With `maxval`, magnitudes above it saturate to it."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 of values just below a power of two can round up; fix the exponent exactly
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, emin)
    quantum = np.exp2(e - mbits)
    r = np.rint(a / quantum) * quantum     # np.rint: round half to even; a/quantum is exact
    if maxval is not None:
        r = np.minimum(r, maxval)
    return np.copysign(r, v)


def bf16_round(v):
    """Round fp64 values to the nearest bf16 value (ties to even)."""
    return round_to_grid(v, 7, -126, None)


def bf16_from_bits(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_to_bits(v) -> np.ndarray:
    """Bits of values that are already exactly bf16."""
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _code_of_value(q, fmt: str) -> np.ndarray:
    """Element code of values already on the element grid (sign bit kept for zeros)."""
    table = E2M1_TABLE if fmt == "e2m1" else E4M3_TABLE
    sign_bit = 8 if fmt == "e2m1" else 0x80
    mags = np.abs(table[: sign_bit])               # codes 0..sign_bit-1 are the non-negative ones
    a = np.abs(q)
    idx = np.searchsorted(mags[np.isfinite(mags)], a)
    assert np.all(mags[idx] == a), "value not on the element grid"
    return (idx | np.where(np.signbit(q), sign_bit, 0)).astype(np.uint8)


def mx_quantize(v, fmt: str, block: int = 32):
    """Encode fp64 values (last axis a multiple of `block`) as MX.
    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/block])."""
    mbits, emin, maxval, emax = FORMATS[fmt]
    v = np.asarray(v, np.float64)
    K = v.shape[-1]
    assert K % block == 0
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.abs(vb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    e = np.where(np.exp2(e) > amax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= np.where(amax > 0, amax, 1.0), e + 1, e)
    shared = np.clip(e - emax, -127, 127)
    scale_byte = np.where(amax > 0, shared + 127, 0).astype(np.uint8)
    x = np.where(amax[..., None] > 0, vb / np.exp2(shared)[..., None], vb * 0.0)
    q = round_to_grid(x, mbits, emin, maxval)
    codes = _code_of_value(q, fmt).reshape(v.shape)
    return codes, scale_byte


def mx_dequantize(codes, scale_bytes, fmt: str, block: int = 32) -> np.ndarray:
    """Decode MX (unpacked codes [..., K], scale bytes [..., K/block]) to fp64, exactly."""
    table = E2M1_TABLE if fmt == "e2m1" else E4M3_TABLE
    codes = np.asarray(codes)
    vals = table[codes.astype(np.int64)]
    K = codes.shape[-1]
    vb = vals.reshape(codes.shape[:-1] + (K // block, block))
    return (vb * e8m0_value(scale_bytes)[..., None]).reshape(codes.shape)


def unpack_fp4(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes, element 2i from the low nibble."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_fp4(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_matrix(packed_codes, scale_bytes) -> np.ndarray:
    """Canonical MXFP4 matrix (codes [N, K/2] packed, scales [N, K/32]) -> fp64 [N, K]."""
    return mx_dequantize(unpack_fp4(packed_codes), scale_bytes, "e2m1")

"""Pins of the oracle's MX / bf16 codec against the format definitions and torch's casts."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mx

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")))


def test_e2m1_table_matches_spec():
    mags = GOLD["e2m1_magnitudes_by_code"]
    for c in range(8):
        assert mx.E2M1_TABLE[c] == mags[c]
        assert mx.E2M1_TABLE[c + 8] == -mags[c]
        assert np.signbit(mx.E2M1_TABLE[c + 8])          # code 8 is -0


def test_e4m3_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = mx.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2                                  # S.1111.111 only
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))
    assert np.nanmax(ours) == GOLD["e4m3_max_normal"]
    assert ours[8] == GOLD["e4m3_min_normal"] and ours[1] == GOLD["e4m3_min_subnormal"]


def test_e8m0():
    assert mx.e8m0_value(127) == 1.0
    assert mx.e8m0_value(0) == 2.0 ** -127
    assert mx.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(mx.e8m0_value(255))


@pytest.mark.parametrize("v,expect", GOLD["e2m1_rne_ties"] + GOLD["e2m1_saturation"])
def test_e2m1_rounding_ties_and_saturation(v, expect):
    q = mx.round_to_grid(np.array([v, -v]), *mx.FORMATS["e2m1"][:3])
    assert q[0] == expect and q[1] == -expect


def test_e4m3_rounding_matches_torch_below_448():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(size=20000) * 50, rng.normal(size=5000) * 1e-2,
                        rng.uniform(-447.9, 447.9, 5000)])
    # include exact midpoints of the E4M3 grid
    g = mx.E4M3_TABLE[:126]
    mids = (g[:-1] + g[1:]) / 2
    v = np.concatenate([v, mids, -mids]).astype(np.float32).astype(np.float64)
    ours = mx.round_to_grid(v, *mx.FORMATS["e4m3"][:3])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    q = mx.round_to_grid(np.array([449.0, 1e6, -470.0]), *mx.FORMATS["e4m3"][:3])
    assert list(q) == [448.0, 448.0, -448.0]


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(size=50000), rng.normal(size=1000) * 1e-30, rng.normal(size=1000) * 1e30])
    v32 = v.astype(np.float32).astype(np.float64)           # torch rounds from fp32
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mx.bf16_round(v32), ref)
    # bit round trip
    bits = mx.bf16_to_bits(ref)
    assert np.array_equal(mx.bf16_from_bits(bits), ref)


def test_mx_scale_selection_examples():
    # e = floor(log2 amax) - emax_elem
    cases = [  # (amax, fmt, expected scale byte)
        (1.0, "e2m1", 127 - 2), (6.0, "e2m1", 127 + 0), (7.99, "e2m1", 127), (8.0, "e2m1", 128),
        (0.75, "e2m1", 127 - 1 - 2), (448.0, "e4m3", 127), (512.0, "e4m3", 128), (1.0, "e4m3", 127 - 8),
    ]
    for amax, fmt, byte in cases:
        v = np.zeros(32)
        v[5] = amax
        v[7] = -amax / 3
        codes, sb = mx.mx_quantize(v, fmt)
        assert sb[0] == byte, (amax, fmt, sb[0], byte)
        deq = mx.mx_dequantize(codes, sb, fmt)
        # largest element lands on the grid's top binade, saturating only above max
        assert deq[5] <= amax and deq[5] >= amax / 2


def test_mx_zero_block_and_signed_zero():
    v = np.zeros((2, 32))
    v[1, 3] = -0.0
    codes, sb = mx.mx_quantize(v, "e2m1")
    assert sb.tolist() == [[0], [0]]
    assert codes[1, 3] == 8 and codes[0, 3] == 0
    # a negative value far below the smallest step rounds to -0 (code 8)
    v = np.zeros(32)
    v[0] = 1.0
    v[1] = -1e-9
    codes, sb = mx.mx_quantize(v, "e2m1")
    assert codes[1] == 8


def test_mx_roundtrip_exact_on_grid():
    rng = np.random.default_rng(2)
    for fmt, table in (("e2m1", mx.E2M1_TABLE), ("e4m3", mx.E4M3_TABLE)):
        finite = np.nonzero(np.isfinite(table))[0]
        codes = rng.choice(finite, size=(64, 128)).astype(np.uint8)
        # force a max-magnitude element in every block so the scale reproduces
        top = int(np.nanargmax(table))
        codes.reshape(64, 4, 32)[:, :, 0] = top
        sbytes = rng.integers(100, 150, size=(64, 4)).astype(np.uint8)
        vals = mx.mx_dequantize(codes, sbytes, fmt)
        c2, s2 = mx.mx_quantize(vals, fmt)
        assert np.array_equal(s2, sbytes)
        assert np.array_equal(mx.mx_dequantize(c2, s2, fmt), vals)


def test_mx_quantize_is_nearest_on_scaled_grid():
    """Brute force: each element is the nearest grid point of V/X (ties aside)."""
    rng = np.random.default_rng(3)
    v = rng.normal(size=(200, 32)) * np.exp2(rng.integers(-10, 10, size=(200, 1)))
    for fmt, table in (("e2m1", mx.E2M1_TABLE), ("e4m3", mx.E4M3_TABLE)):
        codes, sb = mx.mx_quantize(v, fmt)
        X = mx.e8m0_value(sb)
        grid = table[np.isfinite(table)]
        scaled = v / X
        dist = np.abs(scaled[..., None] - grid[None, None, :])
        best = grid[np.argmin(dist, axis=-1)]
        got = mx.mx_dequantize(codes, sb, fmt) / X
        assert np.allclose(np.abs(got), np.abs(best))


def test_fp4_pack_layout():
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16)
    packed = mx.pack_fp4(codes)
    assert packed[0, 0] == 0x10 and packed[0, 7] == 0xFE     # element 2i low nibble
    assert np.array_equal(mx.unpack_fp4(packed), codes)

"""Pins of the Quantile Balancing oracle (oracle/balance.py) against what the reading fixes:
brute force on small inputs, the per-expert count at the cutoff, scale behaviour, and the effect
on a skewed router."""
from __future__ import annotations

import numpy as np

from oracle import balance, layer


def test_quota_rounding():
    assert balance.quota(64, 16, 896) == 1          # 1.14 -> 1
    assert balance.quota(8192, 16, 896) == 146      # 146.29 -> 146
    assert balance.quota(7, 1, 2) == 4              # 3.5 -> 4 (halves up)
    assert balance.quota(3, 4, 1) == 3              # clamped to T
    assert balance.quota(1, 1, 100) == 1            # at least one


def test_brute_force_small():
    rng = np.random.default_rng(0)
    for T, E, k in [(5, 3, 1), (12, 4, 2), (33, 7, 3)]:
        s = rng.random((T, E)).astype(np.float32)
        b = balance.quantile_bias(s, k)
        m = balance.quota(T, k, E)
        for e in range(E):
            col = sorted((float(v) for v in s[:, e]), reverse=True)
            assert b[e] == np.float32(-col[m - 1])


def test_exactly_m_keys_at_or_above_zero_per_expert():
    rng = np.random.default_rng(1)
    T, E, k = 500, 40, 4
    s = rng.random((T, E)).astype(np.float32)  # distinct with probability one
    b = balance.quantile_bias(s, k)
    m = balance.quota(T, k, E)
    counts = ((s + b[None, :]) >= 0).sum(axis=0)
    assert np.all(counts == m)


def test_per_expert_scale_and_shift():
    rng = np.random.default_rng(2)
    s = rng.random((64, 8)).astype(np.float32)
    b = balance.quantile_bias(s, 2)
    s2 = s.copy()
    s2[:, 3] *= 2.0      # exact in fp32: the cutoff doubles
    s2[:, 5] += 0.25     # the cutoff moves with the shift (one fp32 rounding of each value)
    b2 = balance.quantile_bias(s2, 2)
    assert b2[3] == 2.0 * b[3]
    assert b2[5] == -(np.float32(-b[5]) + np.float32(0.25))
    keep = [e for e in range(8) if e not in (3, 5)]
    assert np.array_equal(b2[keep], b[keep])


def test_balances_a_skewed_router():
    """Scores with a strong per-expert offset (hot experts): the biased top-k load has a far smaller
    max/mean than the unbiased one."""
    rng = np.random.default_rng(3)
    T, E, k = 2048, 64, 4
    offset = np.linspace(0.0, 3.0, E)
    s = layer.sigmoid(rng.standard_normal((T, E)) + offset[None, :]).astype(np.float32)
    b = balance.quantile_bias(s, k)

    def load(bias):
        idx = layer.select_topk(s.astype(np.float64), bias.astype(np.float64), k).idx
        c = np.bincount(idx.reshape(-1), minlength=E)
        return c.max() / c.mean()

    before, after = load(np.zeros(E, np.float32)), load(b)
    assert before > 4.0 and after < 1.6, (before, after)

"""Quantile Balancing: the router bias b from per-expert router-score quantiles.

TEST INFRASTRUCTURE (see the package docstring).

Sources: "Serving K3, 01 architecture" (the hot-expert paragraph: expert allocation
derived from router-score quantiles, aimed at the tail of the load distribution)
and "Kimi K3: architectural innovations", section "A router decision is also a
scheduling decision" (rank-based calibration: allocation thresholds follow the
observed score distribution, with no feedback knob). The pages give no formula.

Reading taken (plain, rank-based): over a calibration batch of T tokens, expert e's
cutoff c_e is its m-th largest score, m = round(T k / E) (halves rounded up,
clamped to [1, T]): the expert's share of the batch if the load were even. The bias
is b_e = -c_e, so the key s + b of eq. 13 is >= 0 for exactly the m tokens at or
above expert e's cutoff (ties aside): every expert's threshold sits at the same
quantile of its own score distribution. The cutoff is a selection, so b is an
fp32 value exactly.
"""
from __future__ import annotations

import numpy as np


def quota(T: int, k: int, E: int) -> int:
    """m = round(T k / E), halves up, within [1, T]."""
    return int(min(T, max(1, (2 * T * k + E) // (2 * E))))


def quantile_bias(scores: np.ndarray, k: int) -> np.ndarray:
    """b [E] (fp32 values) from fp32 router scores [T, E]: b_e = -(m-th largest of scores[:, e])."""
    s = np.asarray(scores, dtype=np.float32)
    T, E = s.shape
    m = quota(T, k, E)
    desc = -np.sort(-s, axis=0)  # each column in descending order
    return (-desc[m - 1, :]).astype(np.float32)

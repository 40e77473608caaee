"""Reference states for a KV cache whose rows repeat with a period (test helper).

When key row t and value row t of a sequence are row t mod P of a pattern, the
state definition of a key range (max, sum of exp, v_scale-weighted sum of
values) only needs, for every residue r, how many keys of the range have
t mod P = r.  Grouping equal terms this way is exact, and it makes the
reference affordable at millions of keys.  It is pinned against the oracle's
own range states on small contexts by a CPU test.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import e4m3


def residue_counts(lo: int, hi: int, period: int) -> np.ndarray:
    """n[r] = #{t in [lo, hi) : t mod period = r}."""
    r = np.arange(period)

    def upto(x):   # keys t <= x with t mod period = r
        return np.where(x >= r, (x - r) // period + 1, 0)
    if hi <= lo:
        return np.zeros(period, dtype=np.int64)
    return upto(hi - 1) - upto(lo - 1)


class Periodic:
    """Scores and values of one sequence whose K/V rows repeat with `period`."""

    def __init__(self, q_b, k_pattern, v_pattern, k_scale, v_scale, softmax_scale):
        self.period = k_pattern.shape[0]
        c = float(np.float64(softmax_scale) * np.float64(k_scale))
        self.k_hat = e4m3.decode(k_pattern)                 # [P, D]
        self.v_hat = e4m3.decode(v_pattern)
        self.s = (q_b.astype(np.float64).reshape(-1, q_b.shape[-1]) @ self.k_hat.T) * c   # [rows, P]
        self.vs = float(np.float64(v_scale))

    def range_state(self, row: int, lo: int, hi: int):
        n = residue_counts(lo, hi, self.period)
        if n.sum() == 0:
            return -math.inf, 0.0, np.zeros(self.v_hat.shape[1])
        s = self.s[row]
        m = s[n > 0].max()
        w = n * np.exp(np.where(n > 0, s - m, -np.inf))
        return m, w.sum(), self.vs * (w @ self.v_hat)

    def output(self, row: int, hi: int):
        _, l, o = self.range_state(row, 0, hi)
        return o / l

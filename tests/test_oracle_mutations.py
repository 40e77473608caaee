"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case patches one plausible slip into the oracle -- a wrong exponent bias,
an off-by-one causal mask, a missing value scale, swapped page/slot addressing,
a split boundary shifted by one tile -- and checks that the independent pins
(brute force, closed forms, golden values) then fail.  This shows the pins have
teeth; nothing here touches the HIP path.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import brute, e4m3
from tests.oracle_cases import args, layer_np, rel_err


def _brute_disagrees(lens=(40,), nq=3, d=16, ns=3, S=16, seed=77):
    dat = layer_np(list(lens), nq, seed=seed, head_dim=d)
    a = args(dat)
    out = A.attention(*a)
    m, l, o = A.split_states(*a, num_splits=ns, split_size=S)
    bout, bm, bl, bo = brute.brute_force(*a, num_splits=ns, split_size=S)
    bad = rel_err(out, np.array(bout)) > 1e-12 or rel_err(o, np.array(bo)) > 1e-12 \
        or rel_err(l, np.array(bl)) > 1e-12
    return bad


def test_pins_pass_unmutated():
    assert not _brute_disagrees()


def test_catches_wrong_exponent_bias(monkeypatch):
    wrong = np.array([np.ldexp(1.0, -1) * v for v in e4m3.decode_table()])   # bias 8
    monkeypatch.setattr(e4m3, "_TABLE", wrong)
    assert _brute_disagrees()


def test_catches_off_by_one_causal_mask(monkeypatch):
    real = A.query_positions
    monkeypatch.setattr(A, "query_positions", lambda L, q: real(L, q) - 1 if L > q else real(L, q))
    assert _brute_disagrees()


def test_catches_missing_value_scale(monkeypatch):
    real = A.attention

    def no_vscale(q, k, v, bt, cl, ks, vs, ss):
        return real(q, k, v, bt, cl, ks, 1.0, ss)
    monkeypatch.setattr(A, "attention", no_vscale)
    assert _brute_disagrees()


def test_catches_page_slot_transposition(monkeypatch):
    def swapped(cache, block_row, L):
        bs = cache.shape[1]
        n_pages = -(-L // bs)
        rows = cache[np.asarray(block_row[:n_pages], np.int64)]          # [pages, slots, H, D]
        rows = rows.transpose(1, 0, 2, 3).reshape(n_pages * bs, cache.shape[2], cache.shape[3])
        return rows[:L]
    monkeypatch.setattr(A, "gather_codes", swapped)
    assert _brute_disagrees(lens=(48,))


def test_catches_split_boundary_shift(monkeypatch):
    real = A.split_states

    def shifted(*a, num_splits=80, split_size=0):
        return real(*a, num_splits=num_splits, split_size=split_size + 1 if split_size else 0)
    monkeypatch.setattr(A, "split_states", shifted)
    assert _brute_disagrees()

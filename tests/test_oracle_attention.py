"""Pins for the FP64 attention oracle (CPU only).

Each pin checks the oracle against something other than itself: a pure-Python
brute force with exact rational dot products and torch's E4M3 cast, the exact
re-association identity (any split count combines to the unsplit result),
closed forms, and invariances of the definition.
"""
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import brute, e4m3
from tests.oracle_cases import args, layer_np, rel_err

GOLDEN_SPLIT = os.path.join(os.path.dirname(__file__), "golden", "split_tokens.txt")


# ---------------------------------------------------------------- split-size rule

def test_split_rule_reproduces_pages_3296_split_at_capacity_boundary():
    with open(GOLDEN_SPLIT) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert rows
    for L, S in rows:
        assert A.split_tokens(int(L)) == int(S)


@pytest.mark.parametrize("L", [1, 8, 31, 32, 33, 2559, 2560, 2561, 4096, 32768, 131072, 261887, 261888, 262144])
def test_split_rule_properties(L):
    S = A.split_tokens(L)
    assert S % 32 == 0 and S % 16 == 0
    assert 80 * S >= L            # the 80 splits cover the context
    assert 80 * (S - 32) < L or S == 32   # smallest such multiple of 32


def test_split_counts_at_workload_lengths():
    # Non-empty split counts at the workload lengths (derived from the rule).
    def nonempty(L):
        S = A.split_tokens(L)
        return sum(1 for j in range(80) if j * S < L), S
    assert nonempty(4096) == (64, 64)
    assert nonempty(32768) == (79, 416)
    assert nonempty(131072) == (79, 1664)
    n, S = nonempty(261888)
    assert (n, S) == (80, 3296) and 261888 - 79 * S == 1504


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    # lens, nq, head_dim, num_splits, split_size
    ([8], 8, 16, 2, 32),
    ([9], 8, 16, 3, 32),
    ([40], 3, 16, 3, 16),
    ([17], 1, 16, 2, 16),
    ([1], 1, 16, 2, 16),
    ([33, 20], 2, 16, 3, 16),
    ([20], 2, 256, 2, 16),
    ([12], 8, 256, 1, 32),
]


@pytest.mark.parametrize("lens,nq,d,ns,S", BRUTE_CASES)
def test_oracle_matches_pure_python_brute_force(lens, nq, d, ns, S):
    dat = layer_np(lens, nq, seed=11 + len(lens) * 7 + nq, head_dim=d)
    a = args(dat)
    out = A.attention(*a)
    m, l, o = A.split_states(*a, num_splits=ns, split_size=S)
    bout, bm, bl, bo = brute.brute_force(*a, num_splits=ns, split_size=S)
    bout, bl, bo = np.array(bout), np.array(bl), np.array(bo)
    bm = np.array(bm)
    assert rel_err(out, bout) <= 1e-12
    assert np.array_equal(np.isinf(m), np.isinf(bm))
    fin = np.isfinite(bm)
    assert np.max(np.abs(m[fin] - bm[fin])) <= 1e-12 * max(1.0, np.max(np.abs(bm[fin])))
    assert rel_err(l, bl) <= 1e-12
    assert rel_err(o, bo) <= 1e-12


# ---------------------------------------------------------------- split invariance

@pytest.mark.parametrize("ns,S", [(1, 0), (2, 0), (3, 0), (7, 0), (80, 0), (80, 64), (40, 128), (1, 4128),
                                  (2, 2048), (128, 32)])
def test_any_split_count_combines_to_unsplit(ns, S):
    dat = layer_np([4096], 8, seed=5)
    a = args(dat)
    if S == 0:
        S = A.split_tokens(4096, ns)
    if ns * S < 4096:
        pytest.skip("split cover too small")
    ref = A.attention(*a)
    m, l, o = A.split_states(*a, num_splits=ns, split_size=S)
    assert rel_err(A.combine(m, l, o), ref) <= 1e-12


def test_split_invariance_with_peaky_keys_and_mixed_batch():
    dat = layer_np([700, 64, 1500], 5, seed=9, key_mix=0.05)
    a = args(dat)
    ref = A.attention(*a)
    m, l, o = A.split_states(*a)
    assert rel_err(A.combine(m, l, o), ref) <= 1e-12


def test_empty_split_states_are_exact():
    # L = 4096 -> S = 64: splits 64..79 are empty for every row.
    dat = layer_np([4096], 8, seed=3)
    m, l, o = A.split_states(*args(dat))
    assert np.all(m[..., 64:] == -np.inf) and np.all(l[..., 64:] == 0) and np.all(o[..., 64:, :] == 0)
    assert np.all(np.isfinite(m[..., :64]))


def test_split_starting_inside_query_window_leaves_early_rows_empty():
    # L = 70, q = 8, S = 32 -> split 2 covers [64, 70): query i sees keys <= 62 + i,
    # so rows i < 2 have an empty split 2 and rows i >= 2 do not.
    dat = layer_np([70], 8, seed=4)
    m, l, o = A.split_states(*args(dat), num_splits=3, split_size=32)
    assert np.all(m[0, :2, :, 2] == -np.inf) and np.all(l[0, :2, :, 2] == 0)
    assert np.all(np.isfinite(m[0, 2:, :, 2]))
    assert np.allclose(l[0, 2:, :, 2] > 0, True)


# ---------------------------------------------------------------- closed forms

def _set_all_tokens(cache, block_row, L, row_codes):
    bs = cache.shape[1]
    for t in range(L):
        cache[block_row[t // bs], t % bs, 0, :] = row_codes


def test_equal_keys_give_uniform_weights():
    dat = layer_np([300], 8, seed=21)
    L = 300
    krow = dat["k_cache"][dat["block_table"][0][0], 0, 0, :].copy()
    _set_all_tokens(dat["k_cache"], dat["block_table"][0], L, krow)
    a = args(dat)
    out = A.attention(*a)
    v_hat = e4m3.decode(A.gather_codes(dat["v_cache"], dat["block_table"][0], L))[:, 0, :]
    pos = A.query_positions(L, 8)
    for i in range(8):
        expect = dat["v_scale"] * v_hat[: pos[i] + 1].mean(axis=0)
        for h in range(6):
            assert rel_err(out[0, i, h], expect) <= 1e-12
    S = 32
    m, l, o = A.split_states(*a, num_splits=10, split_size=S)
    c = dat["softmax_scale"] * dat["k_scale"]
    k_hat = e4m3.decode(krow)
    for i in range(8):
        for h in range(6):
            s0 = c * float(dat["q"][0, i, h].astype(np.float64) @ k_hat)
            for j in range(10):
                n = max(0, min((j + 1) * S, pos[i] + 1) - j * S)
                assert l[0, i, h, j] == pytest.approx(n, rel=1e-13)
                if n:
                    assert m[0, i, h, j] == pytest.approx(s0, rel=1e-13, abs=1e-13)
                else:
                    assert m[0, i, h, j] == -math.inf


def test_equal_values_give_that_value():
    dat = layer_np([500], 6, seed=22)
    L = 500
    vrow = dat["v_cache"][dat["block_table"][0][3], 5, 0, :].copy()
    _set_all_tokens(dat["v_cache"], dat["block_table"][0], L, vrow)
    out = A.attention(*args(dat))
    expect = dat["v_scale"] * e4m3.decode(vrow)
    for i in range(6):
        for h in range(6):
            assert rel_err(out[0, i, h], expect) <= 1e-13


def test_single_key_context():
    dat = layer_np([1], 1, seed=23)
    a = args(dat)
    out = A.attention(*a)
    page = dat["block_table"][0][0]
    v0 = e4m3.decode(dat["v_cache"][page, 0, 0, :])
    k0 = e4m3.decode(dat["k_cache"][page, 0, 0, :])
    for h in range(6):
        assert rel_err(out[0, 0, h], dat["v_scale"] * v0) <= 1e-15
    m, l, o = A.split_states(*a)
    c = dat["softmax_scale"] * dat["k_scale"]
    for h in range(6):
        assert l[0, 0, h, 0] == 1.0
        assert m[0, 0, h, 0] == pytest.approx(c * float(dat["q"][0, 0, h].astype(np.float64) @ k0), rel=1e-14)
        assert np.all(m[0, 0, h, 1:] == -np.inf)


def test_one_dominant_key_selects_its_value():
    dat = layer_np([200], 4, seed=24)
    L = 200
    dat["q"][:] = np.float16(1.0)
    _set_all_tokens(dat["k_cache"], dat["block_table"][0], L, np.zeros(256, np.uint8))
    star = 57
    page = dat["block_table"][0][star // 16]
    dat["k_cache"][page, star % 16, 0, :] = 0x7E            # 448 in every dimension
    out = A.attention(*args(dat))
    v_star = dat["v_scale"] * e4m3.decode(dat["v_cache"][page, star % 16, 0, :])
    for i in range(4):
        for h in range(6):
            assert rel_err(out[0, i, h], v_star) <= 1e-15


# ---------------------------------------------------------------- invariances

def test_block_table_permutation_is_bit_invariant():
    dat = layer_np([777], 8, seed=31)
    ref = A.attention(*args(dat))
    refm, refl, refo = A.split_states(*args(dat))
    rng = np.random.default_rng(0)
    nb = dat["k_cache"].shape[0]
    perm = rng.permutation(nb)                 # physical page p moves to perm[p]
    k2 = np.empty_like(dat["k_cache"])
    v2 = np.empty_like(dat["v_cache"])
    k2[perm] = dat["k_cache"]
    v2[perm] = dat["v_cache"]
    dat2 = dict(dat, k_cache=k2, v_cache=v2, block_table=perm[dat["block_table"]].astype(np.int32))
    assert np.array_equal(A.attention(*args(dat2)), ref)
    m, l, o = A.split_states(*args(dat2))
    assert np.array_equal(m, refm) and np.array_equal(l, refl) and np.array_equal(o, refo)


def test_causal_rows_ignore_later_keys():
    dat = layer_np([100], 8, seed=32)
    base = A.attention(*args(dat))
    # overwrite the key and value at position 95 (= p_3): rows i < 3 must not change
    t = 95
    page = dat["block_table"][0][t // 16]
    dat["k_cache"][page, t % 16, 0, :] = 0x55
    dat["v_cache"][page, t % 16, 0, :] = 0x56
    out = A.attention(*args(dat))
    assert np.array_equal(out[0, :3], base[0, :3])
    assert not np.allclose(out[0, 3:], base[0, 3:])


def test_score_scale_enters_only_as_product():
    dat = layer_np([256], 8, seed=33)
    a = list(args(dat))
    ref = A.attention(*a)
    a[5], a[7] = a[7], a[5]            # swap k_scale and softmax_scale
    assert rel_err(A.attention(*a), ref) <= 1e-15


def test_value_scale_is_linear():
    dat = layer_np([256], 8, seed=34)
    a = list(args(dat))
    ref = A.attention(*a)
    a[6] = a[6] * 4.0
    assert rel_err(A.attention(*a), 4.0 * ref) <= 1e-15


def test_poisoned_unmapped_data_never_reaches_the_oracle():
    dat = layer_np([333], 8, seed=35)
    out = A.attention(*args(dat))
    m, l, o = A.split_states(*args(dat))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(l)) and np.all(np.isfinite(o))


def test_sampled_helpers_match_full_oracle():
    dat = layer_np([2000], 8, seed=36)
    a = args(dat)
    out = A.attention(*a)
    m, l, o = A.split_states(*a)
    rows = [(0, 0), (7, 5), (3, 2)]
    got = A.reference_rows_at(*a, b=0, rows=rows)
    for k, (i, h) in enumerate(rows):
        assert rel_err(got[k], out[0, i, h]) <= 1e-13
    for (i, h, j) in [(0, 0, 0), (7, 5, 79), (4, 1, 39), (2, 3, 62)]:
        mj, lj, oj = A.split_state_at(*a, b=0, i=i, h=h, j=j)
        assert (mj == m[0, i, h, j]) or abs(mj - m[0, i, h, j]) <= 1e-13 * max(1, abs(mj))
        assert lj == pytest.approx(l[0, i, h, j], rel=1e-13, abs=0)
        assert rel_err(oj, o[0, i, h, j]) <= 1e-13 if np.any(oj) else np.all(o[0, i, h, j] == 0)


def test_range_state_matches_brute_force_per_key_states():
    # Per-key states from the pure-Python brute force (split size 1: m = s_t,
    # l = 1, o = v_scale * V_t) merged by hand over arbitrary key ranges must
    # equal the oracle's state of that range (cut at each row's causal bound).
    dat = layer_np([45], 3, seed=41, head_dim=16)
    a = args(dat)
    _, bm, bl, bo = brute.brute_force(*a, num_splits=45, split_size=1)
    bm = np.array(bm)
    bo = np.array(bo)
    pos = A.query_positions(45, 3)
    for (lo, hi) in [(0, 45), (0, 1), (7, 19), (19, 43), (40, 45), (44, 60), (43, 43)]:
        for i in range(3):
            for h in (0, 5):
                m, l, o = A.range_state_at(*a, b=0, i=i, h=h, lo=lo, hi=hi)
                top = min(hi, int(pos[i]) + 1)
                if lo >= top:
                    assert m == -math.inf and l == 0.0 and not np.any(o)
                    continue
                ms = bm[0, i, h, lo:top]
                mref = ms.max()
                w = np.exp(ms - mref)
                assert m == pytest.approx(mref, rel=1e-13, abs=1e-13)
                assert l == pytest.approx(math.fsum(w), rel=1e-12)
                assert rel_err(o, (w[:, None] * bo[0, i, h, lo:top]).sum(0)) <= 1e-12

"""Pins for the QK-stage oracle (CPU only).

The tiled scores are checked against a pure-Python brute force (exact rational
dot products, torch's E4M3 cast, token-by-token block-table walk), a closed
form, the attention oracle (softmax of the visible scores times V is the
attention output), paging invariance and the bound that the FP32 tolerance is
built on.  Planted mistakes in the oracle must make the brute-force pin fail.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import brute, e4m3
from oracle import qk as QK
from tests.oracle_cases import layer_np


def _qk_args(d):
    return (d["q"], d["k_cache"], d["block_table"], d["context_lens"], d["k_scale"], d["softmax_scale"])


def _same(a, b, rtol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if not np.array_equal(np.isnan(a), np.isnan(b)):
        return False
    if not np.array_equal(np.isneginf(a), np.isneginf(b)):
        return False
    fin = np.isfinite(b)
    if not np.array_equal(fin, np.isfinite(a)):
        return False
    if not fin.any():
        return True
    return float(np.max(np.abs(a[fin] - b[fin]))) <= rtol * max(1.0, float(np.max(np.abs(b[fin]))))


QK_CASES = [
    # lens, nq, head_dim, ld
    ([8], 8, 16, 32),
    ([33], 3, 16, 96),
    ([40, 17], 2, 16, 64),
    ([1], 1, 16, 64),
    ([64], 8, 16, 64),
    ([20], 2, 256, 32),
]


@pytest.mark.parametrize("lens,nq,d,ld", QK_CASES)
def test_tiled_scores_match_brute_force(lens, nq, d, ld):
    dat = layer_np(lens, nq, seed=301 + 5 * len(lens) + nq, head_dim=d)
    a = _qk_args(dat)
    got = QK.tiled_scores(*a, ld=ld)
    ref = np.array(brute.brute_scores(*a, ld=ld))
    assert got.shape == ref.shape == (len(lens), 6 * nq, ld)
    assert _same(got, ref)


def test_guard_and_mask_layout():
    # L = 33, q = 3: rows of token i see keys 0..30+i; the second tile ends at 64.
    dat = layer_np([33], 3, seed=5, head_dim=16)
    s = QK.tiled_scores(*_qk_args(dat), ld=96)
    for i in range(3):
        for h in range(6):
            row = s[0, 6 * i + h]
            assert np.all(np.isfinite(row[:31 + i])) and np.all(np.isneginf(row[31 + i:64]))
            assert np.all(np.isnan(row[64:]))


def test_closed_form_unit_keys():
    # Every key code 0x38 decodes to 1.0 and every query entry is 1: s = c * D.
    dat = layer_np([50], 2, seed=9, head_dim=16)
    dat["k_cache"][:] = 0x38
    dat["q"][:] = np.float16(1.0)
    assert e4m3.decode(np.array([0x38], np.uint8))[0] == 1.0
    s = QK.tiled_scores(*_qk_args(dat), ld=64)
    c = float(np.float32(dat["softmax_scale"])) * float(np.float32(dat["k_scale"]))
    for i in range(2):
        vis = s[0, 6 * i:6 * i + 6, :49 + i]
        assert np.all(vis == c * 16)


def test_softmax_of_visible_scores_is_the_attention_output():
    dat = layer_np([70, 45], 4, seed=21, head_dim=16)
    a = _qk_args(dat)
    s = QK.tiled_scores(*a, ld=96)
    out = A.attention(dat["q"], dat["k_cache"], dat["v_cache"], dat["block_table"], dat["context_lens"],
                      dat["k_scale"], dat["v_scale"], dat["softmax_scale"])
    for b, L in enumerate(dat["context_lens"]):
        v_hat = e4m3.decode(A.gather_codes(dat["v_cache"], dat["block_table"][b], int(L)))[:, 0, :]
        for r in range(6 * 4):
            row = s[b, r, :int(L)]
            w = np.exp(row - np.max(row))          # -inf -> 0
            mine = float(np.float32(dat["v_scale"])) * (w @ v_hat) / w.sum()
            np.testing.assert_allclose(mine, out[b, r // 6, r % 6], rtol=1e-12, atol=1e-14)


def test_paging_invariance():
    dat = layer_np([75], 3, seed=31, head_dim=16)
    s0 = QK.tiled_scores(*_qk_args(dat), ld=96)
    nb = dat["k_cache"].shape[0]
    perm = np.random.default_rng(4).permutation(nb)
    moved = dict(dat)
    moved["k_cache"] = np.empty_like(dat["k_cache"])
    moved["k_cache"][perm] = dat["k_cache"]
    moved["block_table"] = perm[dat["block_table"]].astype(np.int32)
    s1 = QK.tiled_scores(*_qk_args(moved), ld=96)
    assert _same(s1, s0, rtol=0.0)


def test_error_scale_bounds_the_scores_and_matches_brute_force():
    dat = layer_np([21], 2, seed=41, head_dim=16)
    a = _qk_args(dat)
    s = QK.tiled_scores(*a, ld=32)
    e = QK.score_error_scale(*a, ld=32)
    fin = np.isfinite(s)
    assert np.all(np.abs(s[fin]) <= e[fin] * (1 + 1e-15))
    # brute force of c * sum |q| |k| at one position per row
    c = float(np.float32(dat["softmax_scale"])) * float(np.float32(dat["k_scale"]))
    kc = dat["k_cache"][dat["block_table"][0, 0], 3, 0, :]
    kvals = brute._decode_codes(kc.tolist())
    for r in range(12):
        qv = dat["q"][0, r // 6, r % 6, :].astype(np.float64)
        want = c * math.fsum(abs(float(x)) * abs(y) for x, y in zip(qv, kvals))
        assert abs(e[0, r, 3] - want) <= 1e-12 * want


# ---------------------------------------------------------------- planted mistakes

def _disagrees(lens=(40,), nq=3, ld=64, seed=77):
    dat = layer_np(list(lens), nq, seed=seed, head_dim=16)
    a = _qk_args(dat)
    return not _same(QK.tiled_scores(*a, ld=ld), np.array(brute.brute_scores(*a, ld=ld)))


def test_qk_pins_pass_unmutated():
    assert not _disagrees()


def test_qk_catches_off_by_one_causal_mask(monkeypatch):
    real = QK.query_positions
    monkeypatch.setattr(QK, "query_positions", lambda L, q: real(L, q) + 1)
    assert _disagrees()


def test_qk_catches_missing_key_scale(monkeypatch):
    real = QK.tiled_scores

    def no_kscale(q, k, bt, cl, ks, ss, ld):
        return real(q, k, bt, cl, 1.0, ss, ld)
    monkeypatch.setattr(QK, "tiled_scores", no_kscale)
    assert _disagrees()


def test_qk_catches_guard_written(monkeypatch):
    monkeypatch.setattr(QK, "TILE_KEYS", 64)   # last tile rounded too far: guard overwritten
    assert _disagrees(lens=(20,), ld=96)


def test_qk_catches_wrong_row_order(monkeypatch):
    real = QK.tiled_scores

    def heads_major(*a, ld):
        s = real(*a, ld=ld)
        B, R, _ = s.shape
        nq = R // 6
        return s.reshape(B, nq, 6, ld).transpose(0, 2, 1, 3).reshape(B, R, ld)
    monkeypatch.setattr(QK, "tiled_scores", heads_major)
    assert _disagrees()


def test_scores_at_agrees_with_tiled_scores():
    dat = layer_np([70, 45], 3, seed=55, head_dim=16)
    a = _qk_args(dat)
    full = QK.tiled_scores(*a, ld=128)
    keys = np.array([0, 1, 31, 32, 44, 45, 63, 64, 69, 70, 95, 96, 127])
    for b in range(2):
        assert _same(QK.scores_at(*a, b=b, keys=keys), full[b][:, keys], rtol=0.0)


def test_tile_major_is_the_documented_index_map():
    dat = layer_np([70], 2, seed=61, head_dim=16)
    s = QK.tiled_scores(*_qk_args(dat), ld=96)
    tm = QK.tile_major(s, 3)
    assert tm.shape == (1, 3, 12, 32)
    for u in range(3):
        for r in range(12):
            for x in (0, 5, 31):
                a, b = tm[0, u, r, x], s[0, r, 32 * u + x]
                assert (np.isnan(a) and np.isnan(b)) or a == b

"""The periodic-cache reference used by the long-context GPU test agrees with
the oracle's plain definition on contexts the oracle handles (CPU only)."""
import numpy as np
import pytest

from long_context_split_amd import synth
from oracle import attention as A
from tests.oracle_cases import args
from tests.periodic_ref import Periodic, residue_counts


def test_residue_counts_brute_force():
    for lo, hi, P in [(0, 0, 5), (0, 1, 5), (3, 17, 5), (7, 7, 3), (10, 123, 16), (0, 1000, 1000), (999, 2001, 1000)]:
        t = np.arange(lo, hi)
        assert np.array_equal(residue_counts(lo, hi, P), np.bincount(t % P, minlength=P)), (lo, hi, P)


@pytest.mark.parametrize("L,nq,P", [(5000, 3, 300), (1000, 8, 1024), (257, 1, 16)])
def test_periodic_reference_matches_oracle(L, nq, P):
    inp = synth.make_periodic_layer(L, nq, P, seed_base=11, device="cpu", scales=(0.1, 0.07))
    d = inp.numpy()
    ref = Periodic(d["q"][0], inp.meta["k_pattern"].numpy(), inp.meta["v_pattern"].numpy(), d["k_scale"],
                   d["v_scale"], d["softmax_scale"])
    out = A.attention(*args(d))
    m, l, o = A.split_states(*args(d))
    S = A.split_tokens(L)
    for i in range(nq):
        p = L - nq + i
        for h in range(6):
            row = 6 * i + h
            np.testing.assert_allclose(ref.output(row, p + 1), out[0, i, h], rtol=1e-12, atol=1e-13)
            for j in range(80):
                mj, lj, oj = ref.range_state(row, j * S, min((j + 1) * S, p + 1))
                if not np.isfinite(m[0, i, h, j]):
                    assert mj == -np.inf and lj == 0.0 and not oj.any()
                    continue
                assert abs(mj - m[0, i, h, j]) <= 1e-12 * max(1.0, abs(mj))
                assert abs(lj - l[0, i, h, j]) <= 1e-11 * lj
                np.testing.assert_allclose(oj, o[0, i, h, j], rtol=1e-11, atol=1e-11 * np.abs(oj).max())


def test_periodic_layer_layout():
    inp = synth.make_periodic_layer(100, 2, 7, seed_base=3, device="cpu")
    d = inp.numpy()
    t = np.arange(100)
    rows = d["k_cache"][d["block_table"][0][t // 16], t % 16, 0]
    assert np.array_equal(rows, inp.meta["k_pattern"].numpy()[t % 7])
    # the rest of the last page is poison
    assert np.all(d["k_cache"][d["block_table"][0][6], 4:] == synth.POISON_CODE)

"""Host-side logic on the CPU: the benchmark's single-GPU contract and the
seeded input generator's layout (no GPU, no kernel launch)."""
import os
import subprocess
import sys

import numpy as np
import pytest

from long_context_split_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workloads_have_the_pages_shapes():
    w = synth.WORKLOADS
    assert w["ctx261888_16layer"]["context"] == 261888 and w["ctx261888_16layer"]["layers"] == 16
    assert w["ctx261888_16layer"]["num_q"] == (8,)
    assert w["ctx261888_smallq_16layer"]["num_q"] == tuple(range(1, 8))
    assert w["ctx131072_peaky_16layer"]["key_mix"] > 0


@pytest.mark.parametrize("lens,nq", [([100], 8), ([700, 33], 3)])
def test_layer_layout(lens, nq):
    inp = synth.make_layer(lens, nq, seed_base=11, device="cpu")
    d = inp.numpy()
    B = len(lens)
    assert d["q"].shape == (B, nq, 6, 256) and d["q"].dtype == np.float16
    assert d["k_cache"].dtype == np.uint8 and d["k_cache"].shape[1:] == (16, 1, 256)
    npg = [-(-L // 16) for L in lens]
    used = np.concatenate([d["block_table"][b, :npg[b]] for b in range(B)])
    assert len(set(used.tolist())) == used.size          # every logical page its own physical page
    for b, L in enumerate(lens):
        rows = d["k_cache"][d["block_table"][b, :npg[b]]].reshape(-1, 256)
        assert not np.any((rows[:L] & 0x7F) == 0x7F)        # no NaN code inside the context
        assert np.all(rows[L:] == synth.POISON_CODE)        # slots past the end are poison
    assert 0.05 <= float(d["k_scale"]) <= 0.2 and 0.05 <= float(d["v_scale"]) <= 0.2


def test_generator_is_deterministic():
    a = synth.make_layer([300], 4, seed_base=5, device="cpu").numpy()
    b = synth.make_layer([300], 4, seed_base=5, device="cpu").numpy()
    for k in ("q", "k_cache", "v_cache", "block_table"):
        assert np.array_equal(a[k], b[k])

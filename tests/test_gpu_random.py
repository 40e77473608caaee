"""Seeded random shapes through the C ABI, element by element against the FP64
oracle (GPU only).

Each case draws a batch of 1-4 sequences, their lengths (from a few keys to
about 14000, so some sequences end inside the first tile and others span
several chunks), q in 1..8, the split count, sometimes a fixed split size,
sometimes a host-side context bound above the longest sequence (which is what
a caller sizing buffers for capacity passes), sometimes a block-table row
longer than needed, and sometimes peaky keys.  Every output and every (row,
split) state of the workspace is compared with the oracle at the tolerances of
tests/parity_util.py.  The draws are fixed by the seed, so a failure names a
reproducible case.
"""
import sys

import numpy as np
import pytest
import torch

from long_context_split_amd import dfv, synth
from tests.parity_util import check_all

pytestmark = pytest.mark.gpu

PAGE = 16


def _cases(n=24, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        nq = int(rng.integers(1, 9))
        lens = []
        for _ in range(B):
            hi = int(rng.choice([64, 3000, 14000]))
            lens.append(int(rng.integers(nq, hi + 1)))
        ns = int(rng.choice([1, 2, 3, 5, 16, 37, 80, 80, 80, 128]))
        bound = max(lens)
        if rng.random() < 0.3:
            bound = min(bound + int(rng.integers(1, 4000)), 16000)
        S = 0
        if rng.random() < 0.3:
            per = -(-bound // ns)
            S = 32 * (-(-per // 32)) * int(rng.integers(1, 3))
        pages = -(-bound // PAGE)
        max_blocks = pages + (int(rng.integers(1, 40)) if rng.random() < 0.3 else 0)
        key_mix = 0.05 if rng.random() < 0.25 else 0.0
        out.append((i, lens, nq, ns, S, bound, max_blocks, key_mix))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_shape(case):
    i, lens, nq, ns, S, bound, max_blocks, key_mix = case
    print(f"[gpu-case] random case {i}: lens={lens} q={nq} ns={ns} S={S} bound={bound} "
          f"max_blocks={max_blocks} key_mix={key_mix}", flush=True)
    sys.stdout.flush()
    inp = synth.make_layer(lens, nq, seed_base=9100 + i, device="cuda", max_blocks=max_blocks, key_mix=key_mix)
    desc = dfv.make_desc(len(lens), nq, max_blocks, bound, num_splits=ns, split_tokens=S,
                         softmax_scale=inp.softmax_scale)
    assert dfv.check(desc) == 0
    ws = dfv.Workspace.allocate(desc)
    dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    res = dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
               ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())
    check_all(res, inp.numpy(), num_splits=ns, split_tokens=S)

"""dfv_attn_noalloc (the entry point that allocates nothing) against dfv_attn,
through the C ABI (GPU only).

Two calls in a row on the library's static scratch, the second with a smaller
input, must give exactly dfv_attn's bytes (the same kernels run on the same
inputs; only where the key-chunk states live differs), and the oracle's
tolerances on the smaller case.
"""
import sys

import numpy as np
import pytest
import torch

from long_context_split_amd import dfv, synth
from tests.parity_util import check_all

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _results(ws):
    torch.cuda.synchronize()
    return dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
                ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())


def test_noalloc_matches_dfv_attn_on_two_calls_in_a_row():
    cases = [(synth.workload_layer("ctx261888_16layer", 2, device="cuda"), "ctx261888 q8 layer 2"),
             (synth.make_layer([5000], 3, seed_base=9900, device="cuda"), "L=5000 q3")]
    for k, (inp, name) in enumerate(cases):
        _note(f"noalloc call {k + 1}: {name}")
        desc = dfv.desc_for(inp)
        assert dfv.scratch_bytes(desc) > 0            # the chunk states do go to scratch
        ref_ws = dfv.Workspace.allocate(desc)
        dfv.run_layer(inp, ref_ws, desc)
        ref = _results(ref_ws)
        ws = dfv.Workspace.allocate(desc)
        for t in (ws.ws_max, ws.ws_sum, ws.ws_num):
            t.fill_(float("nan"))
        ws.out.fill_(float("nan"))
        dfv.attn_noalloc(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, inp.k_scale,
                         inp.v_scale, ws.ws_max, ws.ws_sum, ws.ws_num, ws.out)
        got = _results(ws)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (name, key)
        if k == 1:
            check_all(got, inp.numpy())


def test_noalloc_refuses_a_bad_descriptor_before_any_launch():
    inp = synth.make_layer([100], 8, seed_base=9901, device="cuda")
    desc = dfv.desc_for(inp)
    ws = dfv.Workspace.allocate(desc)
    ws.out.fill_(7.0)
    desc.num_q = 9
    with pytest.raises(dfv.DfvError) as e:
        dfv.attn_noalloc(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, inp.k_scale,
                         inp.v_scale, ws.ws_max, ws.ws_sum, ws.ws_num, ws.out)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert bool((ws.out == 7.0).all())

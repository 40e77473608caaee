"""HIP path vs the FP64 oracle at the workloads' full sizes, element by element
(GPU only; through the C ABI, in the launch configuration the benchmark times).

Every FP16 output and every (row, split) state of the FP32 workspace is
compared with the oracle's unsplit attention and per-split states: the pages
compare output bytes and the full FP32 numerator/max/sum workspaces through
the capacity boundary ("Reduce DFlash2 attention cost and screen exact QK
reuse", Test Plan) and run output and full-workspace checks for q2..q7 there
("Reduce DFlash2 long-context verification decay", Test Plan and Result).
The oracle needs about a second per layer on the host at 261888 keys.
"""
import sys

import numpy as np
import pytest

from long_context_split_amd import dfv, synth
from tests.parity_util import check_all

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(inp):
    import torch
    desc = dfv.desc_for(inp)
    ws = dfv.Workspace.allocate(desc)
    dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    return dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
                ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())


@pytest.mark.parametrize("name,layer,context", [
    ("ctx32768_16layer", 3, None),
    ("ctx131072_peaky_16layer", 11, None),          # peaky keys: output and the full FP32 workspace
    ("ctx261888_16layer", 0, None),
    ("ctx261888_16layer", 15, None),
    ("ctx261888_16layer", 7, 261887),               # one key short of the boundary: ragged page and tile
])
def test_full_size_every_element(name, layer, context):
    _note(f"full size {name} layer {layer} context {context or synth.WORKLOADS[name]['context']}")
    inp = synth.workload_layer(name, layer, device="cuda", context=context)
    res = _run(inp)
    assert np.all(np.isfinite(res["out"]))
    check_all(res, inp.numpy())


@pytest.mark.parametrize("nq", [1, 2, 3, 4, 5, 6, 7])
def test_full_size_small_q_every_element(nq):
    layer = (5 * nq) % 16
    _note(f"full size ctx261888 q={nq} layer {layer}")
    inp = synth.workload_layer("ctx261888_smallq_16layer", layer, num_q=nq, device="cuda")
    res = _run(inp)
    assert np.all(np.isfinite(res["out"]))
    check_all(res, inp.numpy())

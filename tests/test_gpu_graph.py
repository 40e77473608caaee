"""HIP-graph capture of the verification-attention calls (GPU only).

The entry points launch stream-ordered work with no host synchronisation and
no memsets, so a caller can capture them in a graph (the pages replay their
16-layer attention as a captured graph).  Each replay here is preceded by
eager work on the same buffers, and every replay must reproduce the eager
result byte for byte.  The fixed-capacity case captures once with a fixed
split size and context bound and then changes the device-side context
lengths between replays: the launch geometry does not depend on them.
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


def _snapshot(ws):
    return [t.clone() for t in (ws.out, ws.ws_max, ws.ws_sum, ws.ws_num)]


def _same_bytes(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype != torch.float16 else x.view(torch.int16),
                           y.view(torch.uint8) if y.dtype != torch.float16 else y.view(torch.int16))
               for x, y in zip(a, b))


def _poison(ws):
    ws.out.fill_(float("nan"))
    ws.ws_max.fill_(float("nan"))
    ws.ws_sum.fill_(float("nan"))
    ws.ws_num.fill_(float("nan"))


def test_graph_replay_of_three_layers_matches_eager_bytes():
    _note("graph replay, 3 layers of ctx32768_16layer q=8")
    layers = [synth.workload_layer("ctx32768_16layer", i, device="cuda") for i in range(3)]
    desc = dfv.desc_for(layers[0])
    wss = [dfv.Workspace.allocate(desc) for _ in layers]
    for inp, ws in zip(layers, wss):
        dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    ref = [_snapshot(ws) for ws in wss]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for inp, ws in zip(layers, wss):
            dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    for rep in range(3):
        for ws in wss:
            _poison(ws)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, ws in enumerate(wss):
            assert _same_bytes(_snapshot(ws), ref[i]), f"replay {rep}, layer {i}"


def test_fixed_capacity_graph_follows_device_context_lengths():
    cap, S, ns = 4160, 64, 80
    _note(f"fixed-capacity graph: capacity {cap}, split_tokens {S}, batch 2, q=5")
    inp = synth.make_layer([cap, cap - 33], 5, seed_base=7100, device="cuda")
    desc = dfv.make_desc(2, 5, inp.block_table.shape[1], cap, num_splits=ns, split_tokens=S,
                         softmax_scale=inp.softmax_scale)
    ws = dfv.Workspace.allocate(desc)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    eager = dfv.Workspace.allocate(desc)
    for lens in ([cap, cap - 33], [2500, 4100], [5, 777], [cap, 64]):
        inp.context_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        _poison(ws)
        torch.cuda.synchronize()
        graph.replay()
        dfv.run_layer(inp, eager, desc)
        torch.cuda.synchronize()
        assert _same_bytes(_snapshot(ws), _snapshot(eager)), f"lens {lens}"
        res = dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
                   ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())
        d = inp.numpy()
        d["context_lens"] = np.asarray(lens, dtype=np.int32)
        check_all(res, d, num_splits=ns, split_tokens=S)

"""Edge cases of the admitted set on the GPU, through the C ABI (GPU only).

* key chunks longer than one block-table window (64 tiles of 64 keys), with
  and without a reference restart inside them, and a fixed split size;
* the admitted context bound (2^22 keys) on a cache whose rows repeat, where
  every output and workspace element has an affordable exact reference;
* q = 1 at L = 1, and batches of very short contexts;
* K and V made of every finite E4M3 code, at a moderate and a peaky scale;
* canaries around the scratch buffer, which holds the key-chunk states;
* the chunk-merge entry point against the fused call, byte for byte.

The pages check canaries, tails and q1 paths explicitly ("Reduce DFlash2
attention cost and screen exact QK reuse", Test Plan and Test Result; "Reduce
DFlash2 long-context verification decay", Test Plan and Result).
"""
import sys

import numpy as np
import pytest
import torch

from long_context_split_amd import dfv, synth
from oracle import attention as A
from tests.parity_util import check_all, check_out, check_ws
from tests.periodic_ref import Periodic

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _layer(lens, nq, seed, **kw):
    return synth.make_layer(lens, nq, seed_base=seed, device="cuda", **kw)


def _run(inp, num_splits=80, split_tokens=0, scratch=None):
    desc = dfv.desc_for(inp, num_splits=num_splits, split_tokens=split_tokens)
    ws = dfv.Workspace.allocate(desc)
    dfv.attn(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, inp.k_scale, inp.v_scale,
             ws.ws_max, ws.ws_sum, ws.ws_num, ws.scratch if scratch is None else scratch, ws.out)
    torch.cuda.synchronize()
    return dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
                ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())


def _args(d):
    return (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"], d["k_scale"],
            d["v_scale"], d["softmax_scale"])


# ------------------------------------------------------------------ long key chunks

@pytest.mark.parametrize("L,nq,ns,S", [
    (20000, 8, 1, 0),       # 4 chunks of 5000 keys: 79 tiles, block-table windows 0 and 1
    (40000, 3, 1, 0),       # 10000-key chunks: 157 tiles, windows 0, 1, 2 (window 2 reuses the first buffer)
    (40000, 5, 2, 20000),   # fixed split size: 5000-key chunks
])
def test_chunks_longer_than_a_window(L, nq, ns, S):
    _note(f"long chunks L={L} q={nq} ns={ns} S={S}")
    inp = _layer([L], nq, seed=4100 + nq)
    desc = dfv.desc_for(inp, num_splits=ns, split_tokens=S)
    assert dfv.chunks(desc) == 4
    res = _run(inp, num_splits=ns, split_tokens=S)
    check_all(res, inp.numpy(), num_splits=ns, split_tokens=S)


@pytest.mark.parametrize("star", [9000, 25000])
def test_restart_inside_a_long_chunk(star):
    # One split of 40000 keys in 4 chunks of 312-313 32-key tiles: key 9000 lies
    # in block-table window 2 of the first chunk (64-key tiles 128..155), key
    # 25000 in window 1 of the third (which starts at key 20000); its score
    # exceeds every other by ~900 natural-log units, so the chunk's reference
    # max must be raised and the chunk redone.
    _note(f"restart in a long chunk, dominant key at {star}")
    inp = _layer([40000], 4, seed=4200, scales=(0.125, 0.125))
    inp.q.fill_(1.0)
    page = int(inp.block_table[0, star // 16])
    inp.k_cache[page, star % 16, 0, :] = 0x7E
    res = _run(inp, num_splits=1)
    check_all(res, inp.numpy(), num_splits=1)


# ------------------------------------------------------------------ the admitted context bound

def test_context_bound_with_a_periodic_cache():
    L, nq, P = 1 << 22, 2, 1024
    _note(f"context bound L={L} q={nq} (periodic rows, period {P})")
    inp = synth.make_periodic_layer(L, nq, P, seed_base=77, device="cuda", scales=(0.08, 0.11))
    desc = dfv.desc_for(inp)
    assert dfv.check(desc) == 0 and dfv.chunks(desc) == 3
    res = _run(inp)
    d = dict(q=inp.q.cpu().numpy(), k_scale=float(inp.k_scale[0]), v_scale=float(inp.v_scale[0]),
             softmax_scale=inp.softmax_scale)
    ref = Periodic(d["q"][0], inp.meta["k_pattern"].cpu().numpy(), inp.meta["v_pattern"].cpu().numpy(),
                   d["k_scale"], d["v_scale"], d["softmax_scale"])
    S = A.split_tokens(L)
    m = np.empty((1, nq, 6, 80))
    l = np.empty_like(m)
    o = np.empty((1, nq, 6, 80, 256))
    out = np.empty((1, nq, 6, 256))
    for i in range(nq):
        p = L - nq + i
        for h in range(6):
            out[0, i, h] = ref.output(6 * i + h, p + 1)
            for j in range(80):
                m[0, i, h, j], l[0, i, h, j], o[0, i, h, j] = ref.range_state(6 * i + h, j * S,
                                                                              min((j + 1) * S, p + 1))
    check_out(res["out"], out)
    check_ws(res["ws_max"], res["ws_sum"], res["ws_num"], m, l, o)
    # the oracle itself on sampled splits (it reads the cache through the block table)
    full = dict(d, k_cache=inp.k_cache.cpu().numpy(), v_cache=inp.v_cache.cpu().numpy(),
                block_table=inp.block_table.cpu().numpy(), context_lens=inp.context_lens.cpu().numpy())
    for (i, h, j) in [(0, 0, 0), (1, 5, 79), (1, 2, 40)]:
        mj, lj, oj = A.split_state_at(*_args(full), b=0, i=i, h=h, j=j)
        check_ws(res["ws_max"][0, i, h, j][None], res["ws_sum"][0, i, h, j][None],
                 res["ws_num"][0, i, h, j][None], np.array([mj]), np.array([lj]), oj[None])


# ------------------------------------------------------------------ tiny contexts

def test_single_query_single_key():
    _note("q=1 L=1")
    inp = _layer([1], 1, seed=4300)
    res = _run(inp)
    check_all(res, inp.numpy())
    d = inp.numpy()
    v0 = d["v_scale"] * A.e4m3.decode(d["v_cache"][d["block_table"][0, 0], 0, 0])
    check_out(res["out"][0, 0], np.broadcast_to(v0, (6, 256)))
    assert np.all(res["ws_sum"][0, 0, :, 0] == 1.0)
    assert np.all(res["ws_max"][0, 0, :, 1:] == -np.inf) and not res["ws_num"][0, 0, :, 1:].any()


@pytest.mark.parametrize("lens,nq", [([1, 2, 17, 1], 1), ([2, 3, 9], 2), ([8, 8], 8)])
def test_batches_of_tiny_contexts(lens, nq):
    _note(f"tiny batch {lens} q={nq}")
    inp = _layer(lens, nq, seed=4400 + nq)
    check_all(_run(inp), inp.numpy())
    check_all(_run(inp, num_splits=1), inp.numpy(), num_splits=1)


# ------------------------------------------------------------------ every finite E4M3 code

def _all_codes(inp, L):
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.long, device="cuda")
    t = torch.arange(L, device="cuda")[:, None]
    d = torch.arange(256, device="cuda")[None, :]
    idx = torch.where(d < 254, (d + 7 * t) % 254, (3 * t + 127 * (d - 254)) % 254)
    rows = finite[idx].to(torch.uint8)
    pages = inp.block_table[0, torch.arange(L, device="cuda") // 16].long()
    slots = torch.arange(L, device="cuda") % 16
    inp.k_cache[pages, slots, 0, :] = rows
    inp.v_cache[pages, slots, 0, :] = rows.flip(1)


@pytest.mark.parametrize("L,nq,k_scale", [(3000, 8, 0.02), (700, 3, 0.02), (3000, 8, 0.1), (2000, 1, 0.1)])
def test_every_finite_code(L, nq, k_scale):
    # Each K and V row holds all 254 finite codes (a different permutation per
    # row), so every code passes through the decode of both operands; with the
    # larger scale the scores spread over about ten natural-log units per
    # standard deviation, rows are peaky and chunk restarts happen.  (At 0.25
    # the scores reach ~100 units, c * sum_d |Q_d K_d| ~ 130; the FP32 rounding
    # of the score itself then moves exp() by ~1e-5, the sum's whole bound:
    # measured 1.07e-5.)
    _note(f"all E4M3 codes L={L} q={nq} k_scale={k_scale}")
    inp = _layer([L], nq, seed=4500 + L + nq, scales=(k_scale, 1.0 / 448.0))
    _all_codes(inp, L)
    res = _run(inp)
    check_all(res, inp.numpy())


# ------------------------------------------------------------------ scratch canary

@pytest.mark.parametrize("lens,nq", [([20000], 8), ([3000], 2)])
def test_scratch_stays_inside_its_buffer(lens, nq):
    _note(f"scratch canary {lens} q={nq}")
    inp = _layer(lens, nq, seed=4600 + nq)
    desc = dfv.desc_for(inp)
    nbytes = dfv.scratch_bytes(desc)
    assert nbytes > 0
    pad = 4096
    raw = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    res = _run(inp, scratch=raw[pad:pad + nbytes])
    r = raw.cpu().numpy()
    assert np.all(r[:pad] == 0xA5) and np.all(r[-pad:] == 0xA5)
    check_all(res, inp.numpy())


# ------------------------------------------------------------------ the chunk-merge entry point

@pytest.mark.parametrize("lens,nq", [([20000], 8), ([5000, 300, 4096, 77], 5)])
def test_chunk_merge_entry_point_matches_the_fused_call(lens, nq):
    # dfv_attn_split_chunks followed by dfv_attn_combine_chunks gives the bytes
    # of dfv_attn; with four sequences there is one chunk per split and the
    # merge is a copy into the workspace.
    _note(f"split_chunks + combine_chunks {lens} q={nq}")
    inp = _layer(lens, nq, seed=4700 + nq)
    desc = dfv.desc_for(inp)
    ref = _run(inp)
    cm, cl, cn = dfv.chunk_buffers(desc)
    dfv.attn_split_chunks(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens,
                          inp.k_scale, inp.v_scale, cm, cl, cn)
    for with_out in (True, False):
        ws = dfv.Workspace.allocate(desc)
        ws.out.fill_(3.0)
        dfv.attn_combine_chunks(desc, cm, cl, cn, ws.ws_max, ws.ws_sum, ws.ws_num, ws.out if with_out else None)
        torch.cuda.synchronize()
        got = dict(ws_max=ws.ws_max.cpu().numpy(), ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())
        for k, v in got.items():
            assert np.array_equal(v, ref[k]), k
        if with_out:
            assert np.array_equal(ws.out.float().cpu().numpy(), ref["out"])
        else:
            assert bool((ws.out == 3.0).all())

"""HIP path vs the FP64 oracle, element by element, through the C ABI (GPU only).

Inputs come from the seeded synthetic generator; the oracle receives host copies
of the very same arrays.  Sizes are small enough for the oracle to finish in
seconds while spanning many 32-key tiles, several workgroups per split and a
ragged tail.  The workloads' full sizes are compared element by element in
test_gpu_full_size.py.
"""
import sys

import numpy as np
import pytest
import torch

from long_context_split_amd import dfv, synth
from oracle import attention as A
from tests.parity_util import check_all, check_out, check_ws, oracle_all

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(inp, num_splits=80, split_tokens=0, entry="attn"):
    desc = dfv.desc_for(inp, num_splits=num_splits, split_tokens=split_tokens)
    ws = dfv.Workspace.allocate(desc)
    if entry == "attn":
        dfv.run_layer(inp, ws, desc)
    else:
        dfv.attn_split(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens,
                       inp.k_scale, inp.v_scale, ws.ws_max, ws.ws_sum, ws.ws_num, ws.scratch)
        dfv.attn_combine(desc, ws.ws_max, ws.ws_sum, ws.ws_num, ws.out)
    torch.cuda.synchronize()
    res = dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
               ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())
    return res, ws, desc


def _layer(lens, nq, seed, **kw):
    return synth.make_layer(lens, nq, seed_base=seed, device="cuda", **kw)


def test_tiny_workload_full_parity():
    inp = synth.workload_layer("tiny_ctx4096", 0, device="cuda")
    _note("tiny_ctx4096 q8 L=4096")
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())


def test_split_then_combine_entry_points_match_fused_call():
    inp = synth.workload_layer("tiny_ctx4096", 0, device="cuda")
    _note("split+combine vs attn")
    r1, _, _ = _run(inp, entry="attn")
    r2, _, _ = _run(inp, entry="split")
    for k in r1:
        assert np.array_equal(r1[k], r2[k], equal_nan=True), k


@pytest.mark.parametrize("L", [8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 1000, 2561, 2592, 2593])
@pytest.mark.parametrize("nq", [1, 3, 8])
def test_tail_contexts(L, nq):
    if L < nq:
        pytest.skip("context shorter than the query window")
    _note(f"tail L={L} q={nq}")
    inp = _layer([L], nq, seed=1000 + L * 10 + nq)
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())


@pytest.mark.parametrize("nq", [1, 2, 3, 4, 5, 6, 7, 8])
def test_q_sweep(nq):
    _note(f"q sweep q={nq} L=3001")
    inp = _layer([3001], nq, seed=2000 + nq)
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())


@pytest.mark.parametrize("nq,L", [(1, 8192), (2, 32768), (3, 32768), (8, 32768)])
def test_repeated_runs_are_byte_identical(nq, L):
    # Every row block count with chunks of two and three 64-key tiles: a read
    # of a value before it is ready shows up as run-to-run differences.
    _note(f"determinism q={nq} L={L}")
    inp = _layer([L], nq, seed=1200 + nq)
    desc = dfv.desc_for(inp)
    outs = []
    for _ in range(3):
        cb = dfv.chunk_buffers(desc)
        for t in cb:
            t.fill_(7.0)
        dfv.attn_split_chunks(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens,
                              inp.k_scale, inp.v_scale, *cb)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in cb])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("nq", [1, 2])
def test_small_q_full_tiles(nq):
    # 12000 keys in 80 splits: chunks of whole 64-key tiles with no masked key,
    # where a score tile's row max reads the MFMA results directly.
    _note(f"full 64-key tiles q={nq} L=12000")
    inp = _layer([12000], nq, seed=2100 + nq)
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())


@pytest.mark.parametrize("ns,S", [(1, 0), (7, 0), (80, 0), (100, 0), (256, 0), (80, 64), (2, 3296), (80, 3296),
                                  (130, 32)])
def test_split_variants(ns, S):
    # Chunks per split: 4 (1, 2, 7 splits), 3 (80), 2 (100), 1 (130, 256).
    L = 4160
    if S and ns * S < L:
        pytest.skip("splits do not cover the context")
    _note(f"splits ns={ns} S={S} L={L}")
    inp = _layer([L], 8, seed=3000 + ns)
    res, _, _ = _run(inp, num_splits=ns, split_tokens=S)
    check_all(res, inp.numpy(), num_splits=ns, split_tokens=S)


def test_batch_mixed_lengths():
    _note("batch lens [70, 4096, 1000, 8] q=5")
    inp = _layer([70, 4096, 1000, 8], 5, seed=5000, max_blocks=300)
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())


def test_peaky_keys():
    _note("peaky keys L=20000")
    inp = _layer([20000], 8, seed=6000, key_mix=0.05)
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())


@pytest.mark.parametrize("star", [6, 1000, 5000, 5990])
def test_late_dominant_key_forces_reference_restart(star):
    # A key whose score exceeds everything else by ~900 natural-log units; when
    # it is not in a wave's first tile the wave must raise its reference max and
    # redo its tiles.  With S = 96 (L = 6000), splits hold 3 tiles, so only the
    # first-tile waves see it without a restart.
    _note(f"dominant key at {star}")
    inp = _layer([6000], 4, seed=7000, scales=(0.125, 0.125))
    inp.q.fill_(1.0)
    bt = inp.block_table.cpu()
    page = int(bt[0, star // 16])
    inp.k_cache[page, star % 16, 0, :] = 0x7E          # 448 in every dimension
    res, _, _ = _run(inp)
    check_all(res, inp.numpy())
    d = inp.numpy()
    v_star = d["v_scale"] * A.e4m3.decode(d["v_cache"][page, star % 16, 0, :])
    assert np.allclose(res["out"][0, -1, 0], v_star, rtol=2e-3, atol=2e-3)


def test_deterministic_and_paging_invariant():
    _note("determinism + paging")
    inp = _layer([5000], 8, seed=8000)
    r1, _, _ = _run(inp)
    r2, _, _ = _run(inp)
    for k in r1:
        assert np.array_equal(r1[k], r2[k]), k
    # move every physical page to a new place and rewrite the block table
    nb = inp.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(1)).cuda()
    k2 = torch.empty_like(inp.k_cache)
    v2 = torch.empty_like(inp.v_cache)
    k2[perm] = inp.k_cache
    v2[perm] = inp.v_cache
    inp2 = synth.LayerInputs(inp.q, k2, v2, perm[inp.block_table.long()].to(torch.int32), inp.context_lens,
                             inp.k_scale, inp.v_scale, inp.softmax_scale)
    r3, _, _ = _run(inp2)
    for k in r1:
        assert np.array_equal(r1[k], r3[k]), k


def test_outputs_stay_inside_their_buffers():
    _note("canaries")
    inp = _layer([3000], 7, seed=9000)
    desc = dfv.desc_for(inp)
    ws = dfv.Workspace.allocate(desc)
    pad = 4096

    def guarded(t):
        raw = torch.full((t.numel() * t.element_size() + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
        inner = raw[pad:pad + t.numel() * t.element_size()].view(t.dtype).view(t.shape)
        return raw, inner

    outs = {k: guarded(getattr(ws, k)) for k in ("ws_max", "ws_sum", "ws_num", "out")}
    dfv.attn(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, inp.k_scale,
             inp.v_scale, outs["ws_max"][1], outs["ws_sum"][1], outs["ws_num"][1], ws.scratch, outs["out"][1])
    torch.cuda.synchronize()
    for k, (raw, inner) in outs.items():
        r = raw.cpu().numpy()
        assert np.all(r[:pad] == 0xA5) and np.all(r[-pad:] == 0xA5), k
    res = dict(out=outs["out"][1].float().cpu().numpy(), ws_max=outs["ws_max"][1].cpu().numpy(),
               ws_sum=outs["ws_sum"][1].cpu().numpy(), ws_num=outs["ws_num"][1].cpu().numpy())
    check_all(res, inp.numpy())


def test_combine_runs_from_an_oracle_workspace():
    _note("combine from oracle workspace")
    inp = _layer([2500], 8, seed=9100)
    d = inp.numpy()
    out, m, l, o = oracle_all(d)
    desc = dfv.desc_for(inp)
    ws_m = torch.tensor(m, dtype=torch.float32, device="cuda")
    ws_l = torch.tensor(l, dtype=torch.float32, device="cuda")
    ws_o = torch.tensor(o, dtype=torch.float32, device="cuda").contiguous()
    res = torch.empty(1, 8, 6, 256, dtype=torch.float16, device="cuda")
    dfv.attn_combine(desc, ws_m, ws_l, ws_o, res)
    torch.cuda.synchronize()
    check_out(res.float().cpu().numpy(), A.combine(m, l, o))


def test_repeated_calls_reuse_buffers():
    _note("repeated calls")
    inp = _layer([9000], 8, seed=9200)
    desc = dfv.desc_for(inp)
    ws = dfv.Workspace.allocate(desc)
    for _ in range(3):
        dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    res = dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
               ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())
    check_all(res, inp.numpy())


def test_bad_descriptor_is_refused_without_launch():
    inp = _layer([100], 8, seed=9300)
    desc = dfv.desc_for(inp)
    ws = dfv.Workspace.allocate(desc)
    ws.out.fill_(7.0)
    desc.num_q = 9
    with pytest.raises(dfv.DfvError) as e:
        dfv.run_layer(inp, ws, desc)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert bool((ws.out == 7.0).all())


def _chunk_ranges(L, ns, C, split_tokens=0):
    """Key range [lo, hi) of every (split j, chunk c), restating the layout that
    dfv_attn_split_chunks documents: tiles of 32 keys cut per split, then into
    C near-equal runs of whole tiles."""
    S = split_tokens if split_tokens else A.split_tokens(L, ns)
    T = -(-L // 32)
    out = {}
    for j in range(ns):
        a, b = min(j * S // 32, T), min((j + 1) * S // 32, T)
        n = b - a
        for c in range(C):
            out[j, c] = (32 * (a + (c * n) // C), 32 * (a + ((c + 1) * n) // C))
    return out


@pytest.mark.parametrize("lens,nq,ns", [([4096], 8, 80), ([20000], 5, 80), ([1500], 1, 40), ([8192], 1, 80),
                                         ([32768], 2, 80)])
def test_chunk_states_match_oracle_key_ranges(lens, nq, ns):
    inp = _layer(lens, nq, seed=1200 + nq)
    _note(f"split_chunks L={lens} q{nq} ns={ns}")
    desc = dfv.desc_for(inp, num_splits=ns)
    C = dfv.chunks(desc)
    assert C > 1
    cm, cl, cn = dfv.chunk_buffers(desc)
    dfv.attn_split_chunks(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens,
                          inp.k_scale, inp.v_scale, cm, cl, cn)
    torch.cuda.synchronize()
    gm, gl, gn = cm.cpu().numpy(), cl.cpu().numpy(), cn.cpu().numpy()
    d = inp.numpy()
    a = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"], d["k_scale"],
         d["v_scale"], d["softmax_scale"])
    ranges = _chunk_ranges(lens[0], ns, C)
    m = np.empty((1, nq, 6, ns, C))
    l = np.empty_like(m)
    o = np.empty((1, nq, 6, ns, C, 256))
    for i in range(nq):
        for h in range(6):
            for (j, c), (lo, hi) in ranges.items():
                m[0, i, h, j, c], l[0, i, h, j, c], o[0, i, h, j, c] = A.range_state_at(
                    *a, b=0, i=i, h=h, lo=lo, hi=hi)
    check_ws(gm, gl, gn, m, l, o)


def test_many_sequences_of_mixed_lengths():
    # B * NS = 480 > 256: one key chunk per split, many workgroups; lengths from
    # the query window itself to several thousand keys, including ones that end
    # inside a page and inside a 32-key tile.
    lens = [8, 4160, 33, 1000, 2593, 64]
    _note(f"batch of {len(lens)} lengths {lens} q=8")
    inp = _layer(lens, 8, seed=3100)
    res, _, desc = _run(inp)
    assert dfv.chunks(desc) == 1
    check_all(res, inp.numpy(), num_splits=80, split_tokens=0)

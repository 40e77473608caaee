"""Paged E4M3 KV append (dfv_kv_append) vs the oracle, bit for bit (GPU only).

Every finite FP16 value (and +-inf) goes through the kernel at several
per-tensor scales and the whole caches must equal the oracle's byte for byte:
written rows hold the oracle's codes, every other row keeps its previous
bytes, padding slots write nothing.  A NaN input must give a NaN code.  The
last case appends a sequence's q verification tokens and then runs the
attention over the updated cache against the FP64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

from long_context_split_amd import dfv, synth
from oracle import kv_append as KA
from tests.parity_util import check_all

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _append_and_compare(kn, vn, slots, ks, vs, nb, seed):
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 256, (nb, 16, 1, 256), dtype=np.uint8)
    vc = rng.integers(0, 256, (nb, 16, 1, 256), dtype=np.uint8)
    want_k, want_v = KA.append(kn, vn, slots, ks, vs, kc, vc)
    dev = dict(kn=torch.from_numpy(kn).cuda(), vn=torch.from_numpy(vn).cuda(),
               sl=torch.from_numpy(slots).cuda(), kc=torch.from_numpy(kc).cuda(), vc=torch.from_numpy(vc).cuda(),
               ks=torch.tensor([ks], dtype=torch.float32, device="cuda"),
               vs=torch.tensor([vs], dtype=torch.float32, device="cuda"))
    dfv.kv_append(dev["kn"], dev["vn"], dev["sl"], dev["ks"], dev["vs"], dev["kc"], dev["vc"])
    torch.cuda.synchronize()
    got_k, got_v = dev["kc"].cpu().numpy(), dev["vc"].cpu().numpy()
    bad_k = np.argwhere(got_k != want_k)
    bad_v = np.argwhere(got_v != want_v)
    assert bad_k.size == 0, f"K differs at {bad_k[:5].tolist()}"
    assert bad_v.size == 0, f"V differs at {bad_v[:5].tolist()}"


@pytest.mark.parametrize("ks,vs", [(0.0731, 1.0), (0.125, 0.19), (3.0, 0.05)])
def test_every_fp16_value_every_byte(ks, vs):
    _note(f"kv append exhaustive fp16, scales {ks} {vs}")
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allh = allh[~np.isnan(allh)]                               # +-inf kept: they saturate
    pad = (-allh.size) % 256
    allh = np.concatenate([allh, np.zeros(pad, np.float16)])
    n = allh.size // 256
    kn = allh.reshape(n, 1, 256)
    vn = np.ascontiguousarray(kn[::-1])
    nb = 40
    slots = np.random.default_rng(1).permutation(nb * 16)[:n].astype(np.int64)
    _append_and_compare(kn, vn, slots, np.float32(ks), np.float32(vs), nb, seed=2)


def test_padding_slots_write_nothing():
    _note("kv append padding slots")
    rng = np.random.default_rng(5)
    nb, n = 8, 12
    kn = (rng.standard_normal((n, 1, 256)) * 4).astype(np.float16)
    vn = (rng.standard_normal((n, 1, 256)) * 4).astype(np.float16)
    slots = np.array([3, -1, 127, nb * 16, 64, -7, 1 << 40, 65, 0, 100, 101, 2], np.int64)
    _append_and_compare(kn, vn, slots, np.float32(0.1), np.float32(0.09), nb, seed=6)


def test_nan_input_gives_a_nan_code():
    _note("kv append NaN")
    kn = np.zeros((1, 1, 256), np.float16)
    kn[0, 0, 7] = np.nan
    kn[0, 0, 9] = -np.nan
    kc = torch.zeros((2, 16, 1, 256), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    dfv.kv_append(torch.from_numpy(kn).cuda(), torch.from_numpy(kn).cuda(),
                  torch.tensor([17], dtype=torch.int64, device="cuda"), one, one, kc, vc)
    torch.cuda.synchronize()
    row = kc[1, 1, 0].cpu().numpy()
    assert (row[7] & 0x7F) == 0x7F and (row[9] & 0x7F) == 0x7F
    assert np.all(row[np.r_[0:7, 8, 10:256]] == 0)


def test_append_then_attention_matches_oracle():
    _note("kv append then attention")
    L, nq = 3000, 8
    inp = synth.make_layer([L], nq, seed_base=6100, device="cuda")
    rng = np.random.default_rng(9)
    kn = (rng.standard_normal((nq, 1, 256))).astype(np.float16)
    vn = (rng.standard_normal((nq, 1, 256))).astype(np.float16)
    bt = inp.block_table.cpu().numpy()[0]
    pos = np.arange(L - nq, L)
    slots = (bt[pos // 16].astype(np.int64) * 16 + pos % 16)
    d = inp.numpy()
    d["k_cache"], d["v_cache"] = KA.append(kn, vn, slots, d["k_scale"], d["v_scale"], d["k_cache"], d["v_cache"])
    dfv.kv_append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(slots).cuda(),
                  inp.k_scale, inp.v_scale, inp.k_cache, inp.v_cache)
    desc = dfv.desc_for(inp)
    ws = dfv.Workspace.allocate(desc)
    dfv.run_layer(inp, ws, desc)
    torch.cuda.synchronize()
    assert np.array_equal(inp.k_cache.cpu().numpy(), d["k_cache"])
    assert np.array_equal(inp.v_cache.cpu().numpy(), d["v_cache"])
    res = dict(out=ws.out.float().cpu().numpy(), ws_max=ws.ws_max.cpu().numpy(),
               ws_sum=ws.ws_sum.cpu().numpy(), ws_num=ws.ws_num.cpu().numpy())
    check_all(res, d, num_splits=80, split_tokens=0)

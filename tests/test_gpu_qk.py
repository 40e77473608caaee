"""QK stage on its own (dfv_qk_scores) vs the FP64 oracle, through the C ABI (GPU only).

Every score is compared with the oracle: small cases (many 32-key tiles,
ragged tails, several sequences, every q) and two full-size layers (261888
keys, and the peaky 131072-key layer).  The buffer is tile-major ([B][tile][6q][32]); the guard
tiles past each sequence's last tile are filled with a canary bit pattern
before the call and must still hold it afterwards.

Tolerance: the kernel forms each score as an FP32-accumulated sum of 256
exact FP16 x FP16 products, then multiplies by c in FP32.  For any summation
order the error is at most 256 * 2^-24 * sum_d |Q_d K_d| (times c), plus one
rounding of the product by c (2^-24 |s|) and of c itself (2^-24 |s|), so
  |s_gpu - s_ref| <= 2^-16 * c * sum_d |Q_d K_d| + 2^-22 * |s_ref|.
Masked positions must be exactly -inf and unmasked ones finite.
"""
import sys

import numpy as np
import pytest
import torch

from long_context_split_amd import dfv, synth
from oracle import qk as QK

pytestmark = pytest.mark.gpu

CANARY = np.int32(0x7FBADBAD)   # a NaN bit pattern no kernel result has


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(inp, tiles=None):
    """Scores in the logical [B][6q][32 * tiles] order (a view of the tile-major buffer)."""
    desc = dfv.desc_for(inp)
    tiles = tiles or dfv.qk_tiles(desc)
    B, nq = inp.q.shape[:2]
    buf = torch.empty((B, tiles, 6 * nq, 32), dtype=torch.float32, device="cuda")
    buf.view(torch.int32).fill_(int(CANARY))
    dfv.qk_scores(desc, inp.q, inp.k_cache, inp.block_table, inp.context_lens, inp.k_scale, buf, tiles)
    torch.cuda.synchronize()
    logical = buf.permute(0, 2, 1, 3).reshape(B, 6 * nq, 32 * tiles)
    return logical, buf, desc, 32 * tiles


def _check(got, ref, err):
    """got float32 array; ref FP64 with -inf masks and NaN for guard positions; err = c*sum|qk|."""
    bits = got.view(np.int32)
    guard = np.isnan(ref)
    assert np.all(bits[guard] == CANARY), "guard region written"
    masked = np.isneginf(ref)
    assert np.all(np.isneginf(got[masked])), "masked score not -inf"
    vis = np.isfinite(ref)
    assert np.all(np.isfinite(got[vis])), "visible score not finite"
    d = np.abs(got[vis].astype(np.float64) - ref[vis])
    tol = 2.0 ** -16 * err[vis] + 2.0 ** -22 * np.abs(ref[vis])
    worst = float(np.max(d / np.maximum(tol, 1e-300))) if d.size else 0.0
    assert worst <= 1.0, f"score error {worst:.3f} x tolerance"


def _oracle(inp, ld):
    d = inp.numpy()
    a = (d["q"], d["k_cache"], d["block_table"], d["context_lens"], d["k_scale"], d["softmax_scale"])
    return QK.tiled_scores(*a, ld=ld), QK.score_error_scale(*a, ld=ld)


@pytest.mark.parametrize("lens,nq", [([4096], 8), ([1000], 8), ([777], 3), ([65], 1), ([8], 8),
                                     ([3000, 1234], 5), ([33, 2049, 512], 2), ([16], 6), ([31], 7)])
def test_every_score_matches_oracle(lens, nq):
    _note(f"qk scores lens={lens} q={nq}")
    inp = synth.make_layer(lens, nq, seed_base=5100 + nq + len(lens), device="cuda")
    scores, _, desc, ld = _run(inp)
    ref, err = _oracle(inp, ld)
    _check(scores.cpu().numpy(), ref, err)


def test_extra_capacity_keeps_the_guard_tiles():
    _note("qk scores with capacity past the last tile")
    inp = synth.make_layer([1000, 300], 4, seed_base=5201, device="cuda")
    scores, _, desc, ld = _run(inp, tiles=32 + 3)
    ref, err = _oracle(inp, ld)
    _check(scores.cpu().numpy(), ref, err)


def test_peaky_keys_scores():
    _note("qk scores, peaky keys")
    inp = synth.make_layer([5000], 8, seed_base=5301, device="cuda", key_mix=0.05)
    scores, _, desc, ld = _run(inp)
    ref, err = _oracle(inp, ld)
    _check(scores.cpu().numpy(), ref, err)


def test_deterministic_and_graph_capturable():
    _note("qk scores: repeat and graph replay")
    inp = synth.make_layer([4100, 900], 8, seed_base=5401, device="cuda")
    _, b1, desc, _ = _run(inp)
    _, b2, _, _ = _run(inp)
    assert torch.equal(b1.view(torch.int32), b2.view(torch.int32))
    out = torch.empty_like(b1)
    tiles = b1.shape[1]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dfv.qk_scores(desc, inp.q, inp.k_cache, inp.block_table, inp.context_lens, inp.k_scale, out, tiles)
    for _ in range(3):
        out.view(torch.int32).fill_(int(CANARY))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), b1.view(torch.int32))


@pytest.mark.parametrize("name,layer", [("ctx261888_16layer", 0), ("ctx131072_peaky_16layer", 5)])
def test_full_size_every_score(name, layer):
    # Every FP32 score of a full-size layer (48 rows x 261888 or 131072 keys)
    # against the FP64 oracle, with the masks, in the launch configuration the
    # bench times.
    _note(f"qk scores full size {name} layer {layer}, every score")
    inp = synth.workload_layer(name, layer, device="cuda")
    scores, _, desc, ld = _run(inp)
    got = scores.cpu().numpy()
    ref, err = _oracle(inp, ld)
    _check(got, ref, err)
    L = int(inp.context_lens[0])
    nq = inp.q.shape[1]
    for r in range(6 * nq):   # row r = 6i + h sees keys 0 .. L - q + i, -inf after that
        lim = L - nq + r // 6
        assert np.all(np.isfinite(got[0, r, :lim + 1]))
        assert np.all(np.isneginf(got[0, r, lim + 1:]))

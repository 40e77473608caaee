"""FP64 oracle for the QK stage on its own: every tiled score of every query row.

Test infrastructure only (see the package docstring for who may use it).

What is computed, restated from the pages.  The pages time a QK producer by
itself, without softmax, PV or the split merge, and check it before timing by
comparing every FP32 tiled score and every guard tile with a frozen producer
([#589] Purpose: private QK producers that reuse each K fragment across the
three 16-row products; [#589] Test Plan: independent QK compared score by
score, guard tiles included).  The scores are the ones the attention's
softmax takes:

  s[b, r, t] = c * <Q[b, i, h, :], K[t, :]>,   r = 6 i + h,   c = softmax_scale * k_scale,

with K the E4M3-decoded key row of token t read through the block table.
Readings taken here (the pages name the check but not the layout):

* Keys are produced in whole 32-key tiles (the 32-key update tile of [#587]
  Implementation).  A tile is written if it starts inside the context.  Inside
  a written tile, keys the row must not see (t > p_i, causal) and keys past the
  context (t >= L_b) hold -inf, as in the attention's masked softmax input.
* Guard tiles are the tiles from ceil(L_b / 32) on, up to the buffer's tile
  capacity: nothing is written there.  The functions here return NaN at those
  positions, meaning "must still hold the caller's canary".
* Values are indexed logically as s[b][r][t] (r = 6 i + h) with a row length
  ld = 32 * capacity; the buffer itself is tile-major, [b][t // 32][r][t % 32]
  (each tile one contiguous block), which :func:`tile_major` produces.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .attention import TILE_KEYS, gather_codes, query_positions


def tiled_scores(q, k_cache, block_table, context_lens, k_scale, softmax_scale, ld: int):
    """FP64 scores [B, 6q, ld] with -inf masks and NaN at the guard positions.

    q float16 [B, nq, Hq, D]; k_cache uint8 [num_blocks, 16, Hkv, D];
    block_table int32 [B, max_blocks]; context_lens int32 [B].
    """
    B, nq, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    c = float(np.float32(softmax_scale)) * float(np.float32(k_scale))
    out = np.full((B, nq * hq, ld), np.nan, dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        end = TILE_KEYS * (-(-L // TILE_KEYS))
        if end > ld:
            raise ValueError("row stride shorter than the last tile")
        pos = query_positions(L, nq)
        k_hat = e4m3.decode(gather_codes(k_cache, block_table[b], L))   # [L, Hkv, D]
        qb = q[b].astype(np.float64)
        for i in range(nq):
            for h in range(hq):
                r = i * hq + h
                s = (k_hat[:, h // group, :] @ qb[i, h, :]) * c           # [L]
                s[pos[i] + 1:] = -np.inf
                out[b, r, :L] = s
                out[b, r, L:end] = -np.inf
    return out


def score_error_scale(q, k_cache, block_table, context_lens, k_scale, softmax_scale, ld: int):
    """c * sum_d |Q[d]| |K[t, d]| at every written position (0 elsewhere).

    The FP32 rounding error of a 256-term dot product accumulated in any order
    is bounded by a small multiple of 2^-24 times this sum, which is what the
    score tolerance is built on.
    """
    B, nq, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    c = float(np.float32(softmax_scale)) * float(np.float32(k_scale))
    out = np.zeros((B, nq * hq, ld), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        k_abs = np.abs(e4m3.decode(gather_codes(k_cache, block_table[b], L)))
        qb = np.abs(q[b].astype(np.float64))
        for i in range(nq):
            for h in range(hq):
                out[b, i * hq + h, :L] = (k_abs[:, h // group, :] @ qb[i, h, :]) * c
    return out


def scores_at(q, k_cache, block_table, context_lens, k_scale, softmax_scale, b: int, keys):
    """FP64 scores [6q, len(keys)] of sequence b at the given key positions.

    Same definition and masks as :func:`tiled_scores` (-inf where the row must
    not look, NaN at guard positions), evaluated only where asked, so that
    full-length contexts can be checked at sampled keys.
    """
    nq, hq, d = q.shape[1:]
    hkv = k_cache.shape[2]
    group = hq // hkv
    c = float(np.float32(softmax_scale)) * float(np.float32(k_scale))
    L = int(context_lens[b])
    end = TILE_KEYS * (-(-L // TILE_KEYS))
    keys = np.asarray(keys, dtype=np.int64)
    pos = query_positions(L, nq)
    out = np.full((nq * hq, keys.size), np.nan, dtype=np.float64)
    inside = keys < L
    block_size = k_cache.shape[1]
    pages = np.asarray(block_table[b], dtype=np.int64)[keys[inside] // block_size]
    k_hat = e4m3.decode(k_cache[pages, keys[inside] % block_size])          # [n, Hkv, D]
    qb = q[b].astype(np.float64)
    for i in range(nq):
        for h in range(hq):
            r = i * hq + h
            row = np.full(keys.size, np.nan)
            row[inside] = (k_hat[:, h // group, :] @ qb[i, h, :]) * c
            row[(keys < end) & (keys > pos[i])] = -np.inf
            out[r] = row
    return out


def tile_major(s, tiles_per_seq: int):
    """Rearrange logical scores [B, R, 32 * tiles_per_seq] into the buffer layout
    [B, tiles_per_seq, R, 32] (element [b][u][r][x] is key 32u + x of row r).
    A pure index permutation: no arithmetic."""
    B, R, ld = s.shape
    if ld != 32 * tiles_per_seq:
        raise ValueError("logical row length must be 32 * tiles_per_seq")
    return s.reshape(B, R, tiles_per_seq, 32).transpose(0, 2, 1, 3)

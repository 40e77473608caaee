"""FP64 oracle for grouped E4M3 verification attention with 80 logical splits.

Test infrastructure only (see the package docstring for who may use it).

What is computed, restated from the pages:

* q draft-verification query tokens (q8 in the pages' runs) with six FP16 query
  heads sharing one KV head, head dimension 256, attend over a paged KV cache
  held in E4M3 ([#589] Test Plan; [#556] Test Plan).  The query tokens are the
  last q positions of the context and are causal among themselves, so query
  token i (0-based) at position p_i = L - q + i sees keys 0..p_i.
* The context is cut into 80 logical splits ([#587] Implementation; [#589]
  Purpose); each split keeps an FP32 running max, a compensated sum and an FP32
  numerator, and a combine kernel merges the splits ([#589] Test Result).  The
  full per-split (numerator, max, sum) workspace is itself an output that the
  pages compare ([#589] Test Plan).
* The split size at the pages' capacity boundary (261888 context tokens) is
  3296 tokens ([#589] Test Plan, "page3296"; [#587] Purpose for the 261888
  boundary).  Reading taken here: S = 32 * ceil(ceil(L / 80) / 32), which gives
  3296 at both 261888 and 262144 and is a multiple of the 32-key online-update
  tile ([#587] Implementation).  An explicit fixed S may be passed instead.

Because merging per-split softmax states by log-sum-exp is an exact
re-association, the merged result *is* plain softmax attention:

  out[b,i,h,:] = sum_{t<=p_i} softmax_t(c * <Q[b,i,h,:], K[t,:]>) * v_scale * V[t,:]

with c = softmax_scale * k_scale and K, V the E4M3-decoded cache rows.  Split j
of row (b,i,h) covers keys [j*S, min((j+1)*S, p_i+1)); its state is

  m_j = max_t s_t,  l_j = sum_t exp(s_t - m_j),  o_j = v_scale * sum_t exp(s_t - m_j) V[t,:]

and an empty range gives (m, l, o) = (-inf, 0, 0).  m is in natural-log units of
the scaled score; v_scale is inside the numerator.  These are readings of the
pages (which name the state but not its units); they are listed with the other
readings in the design notes.

Array conventions (shared with the synthetic input generator, not with the HIP
path's code):

  q            float16 [B, nq, Hq, D]
  k_cache      uint8   [num_blocks, block_size, Hkv, D]   (E4M3 codes)
  v_cache      uint8   [num_blocks, block_size, Hkv, D]
  block_table  int32   [B, max_blocks]
  context_lens int32   [B]             (L_b, including the nq query tokens)
  k_scale, v_scale     float scalars (per layer)
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3

NUM_SPLITS = 80
TILE_KEYS = 32


def split_tokens(context_len: int, num_splits: int = NUM_SPLITS, tile: int = TILE_KEYS) -> int:
    """Split size S = tile * ceil(ceil(L / num_splits) / tile).

    Reading of the pages' "page3296" split at the 261888-token boundary
    ([#589] Test Plan) with the 32-key update tile ([#587] Implementation).
    """
    if context_len < 1:
        raise ValueError("context length must be positive")
    per_split = -(-context_len // num_splits)
    return tile * (-(-per_split // tile))


def query_positions(context_len: int, num_q: int) -> np.ndarray:
    """Positions p_i = L - q + i of the q causal query tokens (the last q of L)."""
    if not 1 <= num_q <= context_len:
        raise ValueError("need 1 <= q <= L")
    return np.arange(context_len - num_q, context_len, dtype=np.int64)


def gather_codes(cache: np.ndarray, block_row: np.ndarray, context_len: int) -> np.ndarray:
    """Logical token-major codes [L, Hkv, D] of one sequence, read through its block table.

    Token t lives in page block_row[t // block_size], slot t % block_size.
    """
    block_size = cache.shape[1]
    n_pages = -(-context_len // block_size)
    pages = np.asarray(block_row[:n_pages], dtype=np.int64)
    rows = cache[pages]                                   # [n_pages, block_size, Hkv, D]
    rows = rows.reshape(n_pages * block_size, cache.shape[2], cache.shape[3])
    return rows[:context_len]


def _scores(q_b: np.ndarray, k_hat: np.ndarray, c: float) -> np.ndarray:
    """s[i, h, t] = c * <Q[i,h,:], K[t, kvh(h), :]> in float64.

    Head h reads KV head h // (Hq // Hkv) (grouped-query mapping; with Hkv = 1
    every query head reads the single KV head).
    """
    nq, hq, d = q_b.shape
    hkv = k_hat.shape[1]
    group = hq // hkv
    out = np.empty((nq, hq, k_hat.shape[0]), dtype=np.float64)
    for h in range(hq):
        kvh = h // group
        out[:, h, :] = (q_b[:, h, :] @ k_hat[:, kvh, :].T) * c
    return out


def _prepare(q, k_cache, v_cache, block_table, context_lens, b, k_scale):
    L = int(context_lens[b])
    nq = q.shape[1]
    pos = query_positions(L, nq)
    k_hat = e4m3.decode(gather_codes(k_cache, block_table[b], L))
    v_hat = e4m3.decode(gather_codes(v_cache, block_table[b], L))
    q_b = q[b].astype(np.float64)                        # FP16 widened exactly
    return L, pos, k_hat, v_hat, q_b


def _check_shapes(q, k_cache, v_cache, block_table, context_lens):
    if q.dtype != np.float16:
        raise TypeError("q must be float16")
    if k_cache.dtype != np.uint8 or v_cache.dtype != np.uint8:
        raise TypeError("KV caches hold uint8 E4M3 codes")
    if k_cache.shape != v_cache.shape:
        raise ValueError("K and V caches must have the same shape")
    if q.shape[2] % k_cache.shape[2] != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if q.shape[0] != block_table.shape[0] or q.shape[0] != context_lens.shape[0]:
        raise ValueError("batch mismatch")


def attention(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
              softmax_scale) -> np.ndarray:
    """Unsplit causal softmax attention in float64: returns out [B, nq, Hq, D]."""
    _check_shapes(q, k_cache, v_cache, block_table, context_lens)
    c = float(np.float64(softmax_scale) * np.float64(k_scale))
    vs = float(np.float64(v_scale))
    B, nq, hq, d = q.shape
    group = hq // k_cache.shape[2]
    out = np.zeros((B, nq, hq, d), dtype=np.float64)
    for b in range(B):
        L, pos, k_hat, v_hat, q_b = _prepare(q, k_cache, v_cache, block_table, context_lens, b, k_scale)
        s = _scores(q_b, k_hat, c)                           # [nq, hq, L]
        visible = np.arange(L)[None, :] <= pos[:, None]      # [nq, L]
        s = np.where(visible[:, None, :], s, -np.inf)
        m = s.max(axis=2, keepdims=True)
        w = np.exp(s - m)                                    # 0 where masked
        den = w.sum(axis=2)
        for h in range(hq):
            num = w[:, h, :] @ v_hat[:, h // group, :]       # [nq, D]
            out[b, :, h, :] = vs * num / den[:, h:h + 1]
    return out


def split_states(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                 softmax_scale, num_splits: int = NUM_SPLITS, split_size: int = 0):
    """Per-split softmax states (m, l, o) in float64.

    Returns m, l with shape [B, nq, Hq, NS] and o with shape [B, nq, Hq, NS, D].
    ``split_size`` 0 selects the per-sequence rule of :func:`split_tokens`.
    """
    _check_shapes(q, k_cache, v_cache, block_table, context_lens)
    c = float(np.float64(softmax_scale) * np.float64(k_scale))
    vs = float(np.float64(v_scale))
    B, nq, hq, d = q.shape
    group = hq // k_cache.shape[2]
    m = np.full((B, nq, hq, num_splits), -np.inf)
    l = np.zeros((B, nq, hq, num_splits))
    o = np.zeros((B, nq, hq, num_splits, d))
    for b in range(B):
        L, pos, k_hat, v_hat, q_b = _prepare(q, k_cache, v_cache, block_table, context_lens, b, k_scale)
        S = split_size if split_size else split_tokens(L, num_splits)
        if num_splits * S < L:
            raise ValueError("splits do not cover the context")
        s = _scores(q_b, k_hat, c)
        for j in range(num_splits):
            lo = j * S
            for i in range(nq):
                hi = min((j + 1) * S, int(pos[i]) + 1)
                if lo >= hi:
                    continue                                  # empty: (-inf, 0, 0)
                for h in range(hq):
                    seg = s[i, h, lo:hi]
                    mj = seg.max()
                    w = np.exp(seg - mj)
                    m[b, i, h, j] = mj
                    l[b, i, h, j] = w.sum()
                    o[b, i, h, j, :] = vs * (w @ v_hat[lo:hi, h // group, :])
    return m, l, o


def combine(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Merge per-split states: out = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j.

    M is the row max over non-empty splits; empty splits (m = -inf) get weight 0.
    A row with every split empty has no defined output and raises.
    """
    M = m.max(axis=-1, keepdims=True)
    if not np.all(np.isfinite(M)):
        raise ValueError("a row has no visible key in any split")
    w = np.exp(m - M)                                        # exp(-inf) = 0
    num = (w[..., None] * o).sum(axis=-2)
    den = (w * l).sum(axis=-1)
    return num / den[..., None]


def round_fp16(x: np.ndarray) -> np.ndarray:
    """Round float64 to FP16 with round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def reference_rows_at(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                      softmax_scale, b: int, rows):
    """Unsplit attention for selected (i, h) rows of batch b only (for sampled checks at
    large L).  Returns float64 [len(rows), D]."""
    L, pos, k_hat, v_hat, q_b = _prepare(q, k_cache, v_cache, block_table, context_lens, b, k_scale)
    c = float(np.float64(softmax_scale) * np.float64(k_scale))
    vs = float(np.float64(v_scale))
    group = q.shape[2] // k_cache.shape[2]
    res = []
    for i, h in rows:
        n = int(pos[i]) + 1
        s = (k_hat[:n, h // group, :] @ q_b[i, h, :]) * c
        w = np.exp(s - s.max())
        res.append(vs * (w @ v_hat[:n, h // group, :]) / w.sum())
    return np.stack(res)


def range_state_at(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                   softmax_scale, b: int, i: int, h: int, lo: int, hi: int):
    """State (m, l, o[D]) of row (b, i, h) over the keys [lo, hi) it may see, i.e.
    [lo, min(hi, p_i + 1)): the same per-split state definition ([#587]
    Implementation; [#589] Test Plan) applied to an arbitrary key range."""
    L = int(context_lens[b])
    pos = query_positions(L, q.shape[1])
    hi = min(hi, int(pos[i]) + 1)
    d = q.shape[3]
    if lo >= hi:
        return -math.inf, 0.0, np.zeros(d)
    block_size = k_cache.shape[1]
    group = q.shape[2] // k_cache.shape[2]
    t = np.arange(lo, hi)
    pages = np.asarray(block_table[b], dtype=np.int64)[t // block_size]
    k_hat = e4m3.decode(k_cache[pages, t % block_size, h // group, :])
    v_hat = e4m3.decode(v_cache[pages, t % block_size, h // group, :])
    c = float(np.float64(softmax_scale) * np.float64(k_scale))
    s = (k_hat @ q[b, i, h, :].astype(np.float64)) * c
    mj = s.max()
    w = np.exp(s - mj)
    return mj, w.sum(), float(np.float64(v_scale)) * (w @ v_hat)


def split_state_at(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                   softmax_scale, b: int, i: int, h: int, j: int, num_splits: int = NUM_SPLITS,
                   split_size: int = 0):
    """State (m, l, o[D]) of one (b, i, h, split j), computed on its own (sampled checks)."""
    L = int(context_lens[b])
    S = split_size if split_size else split_tokens(L, num_splits)
    return range_state_at(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                          softmax_scale, b, i, h, j * S, (j + 1) * S)

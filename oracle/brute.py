"""Pure-Python brute force for tiny inputs.  Test infrastructure only.

It recomputes the causal verification attention and the per-split states with
no numpy arithmetic: codes are decoded by torch's own ``float8_e4m3fn`` cast
(a library routine, independent of :mod:`oracle.e4m3`'s table), dot products are
exact rationals (``fractions.Fraction``) rounded once to float, and sums use
``math.fsum``.  It walks token by token through the block table, so it also
pins the page addressing of :func:`oracle.attention.gather_codes`.

Used only to pin :mod:`oracle.attention` on inputs with a few dozen keys.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch


def _decode_codes(codes) -> list:
    t = torch.tensor(list(codes), dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    return [float(x) for x in t.tolist()]


def _token_row(cache, block_row, t, kvh):
    block_size = cache.shape[1]
    page = int(block_row[t // block_size])
    return _decode_codes(cache[page, t % block_size, kvh, :].tolist())


def brute_force(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, softmax_scale,
                num_splits: int, split_size: int):
    """Returns (out, m, l, o) as nested Python lists indexed [b][i][h][...].

    out[b][i][h] is the unsplit result (list of D floats); m/l/o[b][i][h][j] the
    state of split j (m = -inf, l = 0, o = zeros for an empty split).
    """
    B, nq, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    c = Fraction(float(np.float32(softmax_scale))) * Fraction(float(np.float32(k_scale)))
    vs = float(np.float32(v_scale))
    outs, ms, ls, os_ = [], [], [], []
    for b in range(B):
        L = int(context_lens[b])
        krows = {}
        vrows = {}
        for t in range(L):
            for kvh in range(hkv):
                krows[t, kvh] = _token_row(k_cache, block_table[b], t, kvh)
                vrows[t, kvh] = _token_row(v_cache, block_table[b], t, kvh)
        ob, mb, lb, obb = [], [], [], []
        for i in range(nq):
            p_i = L - nq + i
            oi, mi, li, oii = [], [], [], []
            for h in range(hq):
                kvh = h // group
                qv = [Fraction(float(x)) for x in q[b, i, h, :].tolist()]
                s = []
                for t in range(p_i + 1):
                    exact = sum(qv[e] * Fraction(krows[t, kvh][e]) for e in range(d))
                    s.append(float(exact * c))
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                oi.append([vs * math.fsum(w[t] * vrows[t, kvh][e] for t in range(p_i + 1)) / den
                           for e in range(d)])
                mj_list, lj_list, oj_list = [], [], []
                for j in range(num_splits):
                    lo, hi = j * split_size, min((j + 1) * split_size, p_i + 1)
                    if lo >= hi:
                        mj_list.append(-math.inf)
                        lj_list.append(0.0)
                        oj_list.append([0.0] * d)
                        continue
                    seg = s[lo:hi]
                    mj = max(seg)
                    wj = [math.exp(x - mj) for x in seg]
                    mj_list.append(mj)
                    lj_list.append(math.fsum(wj))
                    oj_list.append([vs * math.fsum(wj[t - lo] * vrows[t, kvh][e] for t in range(lo, hi))
                                    for e in range(d)])
                mi.append(mj_list)
                li.append(lj_list)
                oii.append(oj_list)
            ob.append(oi)
            mb.append(mi)
            lb.append(li)
            obb.append(oii)
        outs.append(ob)
        ms.append(mb)
        ls.append(lb)
        os_.append(obb)
    return outs, ms, ls, os_


def brute_scores(q, k_cache, block_table, context_lens, k_scale, softmax_scale, ld: int, tile: int = 32):
    """Scores as nested lists [b][r][t], r = 6i + h, for the QK-stage pins.

    Exact rational dot products rounded once, token by token through the
    block table; a written 32-key tile holds -inf where the row must not look
    (t > p_i or t >= L_b); positions past the last written tile are NaN.
    """
    B, nq, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    c = Fraction(float(np.float32(softmax_scale))) * Fraction(float(np.float32(k_scale)))
    out = []
    for b in range(B):
        L = int(context_lens[b])
        end = tile * ((L + tile - 1) // tile)
        rows_b = []
        for i in range(nq):
            p_i = L - nq + i
            for h in range(hq):
                kvh = h // group
                qv = [Fraction(float(x)) for x in q[b, i, h, :].tolist()]
                row = []
                for t in range(ld):
                    if t >= end:
                        row.append(math.nan)
                    elif t > p_i:
                        row.append(-math.inf)
                    else:
                        kr = _token_row(k_cache, block_table[b], t, kvh)
                        row.append(float(c * sum(qv[e] * Fraction(kr[e]) for e in range(d))))
                rows_b.append(row)
        out.append(rows_b)
    return out

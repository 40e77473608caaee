"""Helpers for comparing the HIP path with the FP64 oracle (tolerances in one place).

Tolerances (written out here, used by every parity test):
  * FP16 output:   |out - ref| <= 2e-3 + 2e-3 * |ref|, element-wise, against the
                   oracle's float64 result before FP16 rounding.
  * split max m:   |dm| <= 1e-5 * max(1, |m|); empty splits (-inf) must match exactly.
  * split sum l:   |dl| <= 1e-5 * l; empty splits exactly 0.
  * numerator o:   per (b, i, h, split) row, max|do| <= 1e-5 * max|o_ref|; empty rows exactly 0.
The 1e-5 relative bound on the FP32 workspace is read element-wise for m and l
and normwise (max-norm) per numerator row, since element-wise relative error
of near-cancelling sums is ill-posed.
"""
import numpy as np

from oracle import attention as A

OUT_ABS = 2e-3
OUT_REL = 2e-3
WS_REL = 1e-5


def oracle_all(d, num_splits=80, split_tokens=0):
    a = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"], d["k_scale"],
         d["v_scale"], d["softmax_scale"])
    out = A.attention(*a)
    m, l, o = A.split_states(*a, num_splits=num_splits, split_size=split_tokens)
    return out, m, l, o


def check_out(out_gpu, ref):
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    assert np.all(np.isfinite(out_gpu)), "non-finite output"
    err = np.abs(out_gpu - ref)
    bound = OUT_ABS + OUT_REL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"output mismatch at {worst}: gpu {out_gpu[worst]} ref {ref[worst]}"


def check_ws(m_gpu, l_gpu, o_gpu, m, l, o):
    m_gpu = np.asarray(m_gpu, np.float64)
    l_gpu = np.asarray(l_gpu, np.float64)
    o_gpu = np.asarray(o_gpu, np.float64)
    empty = ~np.isfinite(m)
    assert np.array_equal(~np.isfinite(m_gpu), empty), "empty-split pattern differs"
    assert np.all(m_gpu[empty] == -np.inf) and np.all(l_gpu[empty] == 0.0)
    assert np.all(o_gpu[empty] == 0.0), "empty split with nonzero numerator"
    full = ~empty
    dm = np.abs(m_gpu[full] - m[full])
    assert np.all(dm <= WS_REL * np.maximum(1.0, np.abs(m[full]))), f"max: worst {dm.max()}"
    dl = np.abs(l_gpu[full] - l[full]) / l[full]
    assert np.all(dl <= WS_REL), f"sum: worst rel {dl.max()}"
    do = np.abs(o_gpu[full] - o[full]).max(axis=-1)
    scale = np.abs(o[full]).max(axis=-1)
    rel = do / np.maximum(scale, 1e-300)
    assert np.all(rel <= WS_REL), f"numerator: worst normwise rel {rel.max()}"


def check_all(res, d, num_splits=80, split_tokens=0):
    out, m, l, o = oracle_all(d, num_splits, split_tokens)
    check_out(res["out"], out)
    check_ws(res["ws_max"], res["ws_sum"], res["ws_num"], m, l, o)

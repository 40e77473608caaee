"""Oracle for the paged E4M3 KV append of the q verification tokens.

Test infrastructure only (see the package docstring for who may use it).

What is computed.  The pages keep the target model's KV cache in E4M3 with
per-tensor scales ([#589] Test Plan; [#556] Test Plan: E4M3 target KV) but do
not spell out how the new tokens' keys and values get there.  Plainest reading,
taken here: each new token's FP16 key and value rows are divided by the
layer's per-tensor scale in FP32 and rounded to the nearest E4M3 value (ties
to an even mantissa), saturating at +-448 (the format's largest finite
magnitude; a value beyond it never becomes NaN), and written to the cache row
of the token's slot: page slot // 16, row slot % 16.  A negative slot is
padding and writes nothing.  NaN stays NaN (code 0x7F with the input's sign).

The rounding decision is taken on the FP32 quotient x / scale (correctly
rounded), the precision the kernel works in.  The encoder below picks the
nearest code from the decode table of :mod:`oracle.e4m3` (itself pinned to
the OCP formula and torch's cast), so it shares no arithmetic with the GPU
path.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

_POS = e4m3.decode_table()[:0x7F].astype(np.float64)   # codes 0x00..0x7E: 0 .. 448, increasing
MAX_FINITE = float(_POS[-1])                            # 448


def _tie_goes_up(hi):
    """At an exact midpoint the even code wins (round half to even)."""
    return hi % 2 == 0


def encode(x) -> np.ndarray:
    """FP32 values -> E4M3 codes (uint8): nearest, ties to even code, saturating."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))
    hi = np.searchsorted(_POS, a, side="left")           # first code with value >= a
    hi = np.clip(hi, 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & _tie_goes_up(hi))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS[hi], hi, code).astype(np.uint8)   # exact hits
    sign = np.signbit(x)
    code = np.where(sign, code | 0x80, code).astype(np.uint8)
    code = np.where(nan, np.where(sign, 0xFF, 0x7F), code).astype(np.uint8)
    return code


def quantize_rows(x_fp16, scale) -> np.ndarray:
    """FP16 rows [..., D] -> E4M3 codes of the FP32 quotient x / scale."""
    q = np.asarray(x_fp16, dtype=np.float16).astype(np.float32) / np.float32(scale)
    return encode(q)


def append(k_new, v_new, slot_mapping, k_scale, v_scale, k_cache, v_cache):
    """Returns updated copies of (k_cache, v_cache).

    k_new, v_new float16 [N, Hkv, D]; slot_mapping int64 [N]; caches uint8
    [num_blocks, 16, Hkv, D].  Slots outside [0, num_blocks * 16) write nothing.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    bs = kc.shape[1]
    kq = quantize_rows(k_new, k_scale)
    vq = quantize_rows(v_new, v_scale)
    for n, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0 or s >= kc.shape[0] * bs:
            continue
        kc[s // bs, s % bs] = kq[n]
        vc[s // bs, s % bs] = vq[n]
    return kc, vc

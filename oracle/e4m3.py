"""OCP E4M3 decode, written from the format definition.  Test infrastructure only.

The pages keep the target KV cache in E4M3 ([#556] Test Plan; [#589] Test Plan)
and decode it with a private lookup table on their hardware ([#589] Purpose).
E4M3 here is the OCP 8-bit floating point format (OCP FP8 spec v1.0): one sign
bit, four exponent bits with bias 7, three mantissa bits, subnormals at exponent
field 0, no infinities, and NaN only for S.1111.111.  The largest finite value is
448 (S.1111.110).

The oracle decodes by table: ``decode_table()[code]`` is the exact value of the
code as a float64 (every E4M3 value is exactly representable in float64).
"""
from __future__ import annotations

import math

import numpy as np

EXP_BIAS = 7
MANT_BITS = 3


def e4m3_value(code: int) -> float:
    """Exact value of one E4M3 code from the OCP formula.

    field e = bits 6..3, field m = bits 2..0, sign = bit 7:
      e == 15 and m == 7 -> NaN (both signs)
      e == 0             -> (-1)^s * 2^(1-bias) * (m / 8)         (subnormal)
      otherwise          -> (-1)^s * 2^(e-bias) * (1 + m / 8)
    """
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code must be a byte")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> MANT_BITS) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m / 8.0, 1 - EXP_BIAS)
    else:
        mag = math.ldexp(1.0 + m / 8.0, e - EXP_BIAS)
    return sign * mag


def decode_table() -> np.ndarray:
    """float64[256] table of every E4M3 code's value (NaN for the two NaN codes)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 E4M3 codes to float64 by table lookup."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return _TABLE[codes]


_TABLE = decode_table()

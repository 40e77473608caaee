"""Pins for the oracle's E4M3 decode table (CPU only)."""
import math
import os

import numpy as np
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_values.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                rows.append((int(code, 16), float(val)))
    return rows


def test_table_matches_torch_float8_e4m3fn_cast_on_all_codes():
    table = e4m3.decode_table()
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_t, nan_l = np.isnan(table), np.isnan(lib)
    assert np.array_equal(nan_t, nan_l)
    assert np.array_equal(table[~nan_t], lib[~nan_l])
    assert np.array_equal(np.signbit(table[~nan_t]), np.signbit(lib[~nan_l]))


def test_table_matches_ocp_spec_values():
    table = e4m3.decode_table()
    for code, val in _golden():
        if math.isnan(val):
            assert math.isnan(table[code]), hex(code)
        else:
            assert table[code] == val and math.copysign(1, table[code]) == math.copysign(1, val), hex(code)


def test_exactly_two_nan_codes_and_symmetric_signs():
    table = e4m3.decode_table()
    assert [c for c in range(256) if math.isnan(table[c])] == [0x7F, 0xFF]
    for c in range(128):
        if c != 0x7F:
            assert table[c | 0x80] == -table[c]


def test_positive_codes_strictly_increasing():
    table = e4m3.decode_table()
    pos = table[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_every_value_fits_fp16_exactly():
    # The HIP path widens E4M3 to FP16 for the matrix cores; the decoded value set
    # must be exactly representable there (a property of the format, checked here).
    table = e4m3.decode_table()
    finite = table[np.isfinite(table)]
    assert np.array_equal(finite.astype(np.float16).astype(np.float64), finite)


def test_decode_rejects_non_uint8():
    import pytest
    with pytest.raises(TypeError):
        e4m3.decode(np.zeros(3, dtype=np.int32))

"""Pins for the E4M3 KV-append oracle (CPU only).

The encoder is checked against torch's own float8_e4m3fn cast (an independent
library routine: round to nearest even) on every value where that cast is
finite, against the decode table by an exhaustive round trip, against the
tie rule at hand-picked midpoints, and against the saturation reading past
448; the append is checked by walking slots one by one.  Planted mistakes in
the encoder must fail these pins.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3
from oracle import kv_append as KA


def _torch_codes(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _fp16_grid():
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    return x[np.isfinite(x)]


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes)
    assert np.array_equal(KA.encode(vals.astype(np.float32)), codes)


@pytest.mark.parametrize("scale", [1.0, 0.125, 0.0731, 0.19, 3.0])
def test_matches_torch_cast_wherever_it_is_finite(scale):
    x = _fp16_grid() / np.float32(scale)
    x = x[np.isfinite(x) & (np.abs(x) < 464.0)]          # 464 = midpoint of 448 and 480: torch overflows to NaN
    assert np.array_equal(KA.encode(x), _torch_codes(x))


def test_matches_torch_on_random_fp32():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) < 464.0]
    assert np.array_equal(KA.encode(x), _torch_codes(x))


def test_ties_go_to_the_even_code():
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A; subnormal step 2^-9
    assert KA.encode(np.float32(1.0625)) == 0x38
    assert KA.encode(np.float32(1.1875)) == 0x3A
    assert KA.encode(np.float32(-1.1875)) == 0xBA
    assert KA.encode(np.float32(2.0 ** -10)) == 0x00          # half the smallest subnormal: to zero (even)
    assert KA.encode(np.float32(3 * 2.0 ** -10)) == 0x02      # between codes 1 and 2: to 2
    assert KA.encode(np.float32(-0.0)) == 0x80


def test_saturation_and_nan():
    big = np.array([448.0, 463.9, 464.0, 480.0, 1e6, np.inf], np.float32)
    assert np.all(KA.encode(big) == 0x7E)
    assert np.all(KA.encode(-big) == 0xFE)
    assert KA.encode(np.float32(np.nan)) == 0x7F


def test_append_writes_each_slot_row_and_nothing_else():
    rng = np.random.default_rng(8)
    nb, bs, D = 6, 16, 256
    kc = rng.integers(0, 256, (nb, bs, 1, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (nb, bs, 1, D), dtype=np.uint8)
    N = 9
    kn = (rng.standard_normal((N, 1, D)) * 3).astype(np.float16)
    vn = (rng.standard_normal((N, 1, D)) * 3).astype(np.float16)
    slots = np.array([0, 17, -1, 95, 40, nb * bs, 41, 15, 64], np.int64)
    ks, vs = np.float32(0.11), np.float32(0.07)
    k2, v2 = KA.append(kn, vn, slots, ks, vs, kc, vc)
    touched = set()
    for n, s in enumerate(slots):
        if 0 <= s < nb * bs:
            page, row = divmod(int(s), bs)
            touched.add((page, row))
            for d in (0, 7, 255):
                assert k2[page, row, 0, d] == _torch_codes([np.float32(kn[n, 0, d]) / ks])[0]
                assert v2[page, row, 0, d] == _torch_codes([np.float32(vn[n, 0, d]) / vs])[0]
    for page in range(nb):
        for row in range(bs):
            if (page, row) not in touched:
                assert np.array_equal(k2[page, row], kc[page, row])
                assert np.array_equal(v2[page, row], vc[page, row])


# ---------------------------------------------------------------- planted mistakes

def _torch_pin_fails():
    x = _fp16_grid() / np.float32(0.125)   # exact quotients: many sit on E4M3 midpoints
    x = x[np.isfinite(x) & (np.abs(x) < 464.0)]
    return not np.array_equal(KA.encode(x), _torch_codes(x))


def test_catches_ties_away_from_zero(monkeypatch):
    monkeypatch.setattr(KA, "_tie_goes_up", lambda hi: np.ones_like(hi, dtype=bool))
    assert _torch_pin_fails()


def test_catches_dropped_sign(monkeypatch):
    monkeypatch.setattr(KA.np, "signbit", lambda x: np.zeros(np.shape(x), dtype=bool))
    assert _torch_pin_fails()


def test_catches_wrong_table(monkeypatch):
    monkeypatch.setattr(KA, "_POS", KA._POS * 2.0)
    assert _torch_pin_fails()

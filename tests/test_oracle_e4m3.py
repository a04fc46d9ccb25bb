"""Pins for the oracle's FP8 e4m3fn codec and absmax quantisation.

The pages fix only "FP8 quantization" at write time (Runway Characters,
abstract); the format is e4m3fn.  The codec is pinned against the OCP FP8
specification's table (tests/golden/e4m3_spec_values.txt), against torch's
CPU float8_e4m3fn conversion (a library routine) on every code and on every
rounding midpoint in range, and against hand-checked ties.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), val))
    return rows


def test_decode_matches_spec_table():
    rows = _golden()
    assert len(rows) >= 20
    for code, val in rows:
        got = e4m3.DECODE_TABLE[code]
        if val == "nan":
            assert math.isnan(got), hex(code)
            continue
        num, den = val.split("/")
        neg = num.startswith("-")
        exp = Fraction(int(num.lstrip("-")), int(den))
        assert Fraction(abs(got)) == exp, hex(code)
        assert math.copysign(1.0, got) == (-1.0 if neg else 1.0), hex(code)


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))
    assert nan.sum() == 2 and np.nanmax(np.abs(ours)) == 448.0


def _torch_encode(x):
    # torch converts float64 through float32, so only float32 inputs are
    # compared (for those its cast is a single rounding).
    x32 = np.asarray(x, dtype=np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64))
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_midpoints_and_grid():
    vals = e4m3.DECODE_TABLE[:127].astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # exact
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    eps = np.concatenate([vals, mids, up, dn, np.nextafter(vals, np.float32(np.inf))])
    eps = eps[eps <= 448.0].astype(np.float64)
    x = np.concatenate([eps, -eps])
    ref = _torch_encode(x)
    ours = e4m3.encode(x)
    # compare decoded values (+0 / -0 both zero)
    assert np.array_equal(e4m3.decode(ref), e4m3.decode(ours))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(123)
    x = rng.uniform(-448, 448, size=200_000) * rng.choice([1.0, 1e-1, 1e-2, 1e-3], size=200_000)
    x = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(e4m3.decode(_torch_encode(x)), e4m3.decode(e4m3.encode(x)))


def test_encode_saturates():
    # torch's cast returns NaN past the rounding range, so saturation is pinned
    # directly from the rule: magnitudes above 448 become 448.
    x = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e6, np.inf, -449.0, -1e9, -np.inf])
    got = e4m3.encode(x)
    assert list(got) == [0x7E] * 7 + [0xFE] * 3


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),          # tie 1.0 | 1.125 -> even 1.0
    (1.1875, 0x3A),          # tie 1.125 | 1.25 -> even 1.25
    (2.0 ** -10, 0x00),      # tie 0 | 2^-9 -> even 0
    (3 * 2.0 ** -10, 0x02),  # tie 2^-9 | 2^-8 -> even 2^-8
    (3 * 2.0 ** -11, 0x01),  # 0.75 * 2^-9 -> nearest 2^-9
    (432.0, 0x7E),           # tie 416 | 448 -> even 448 (0x7E)
    (-1.0625, 0xB8),
])
def test_ties_to_even(x, code):
    assert int(e4m3.encode(np.array([x]))[0]) == code


def test_ulp_distance():
    assert e4m3.ulp_distance(np.uint8(0x00), np.uint8(0x80)) == 0
    assert e4m3.ulp_distance(np.uint8(0x01), np.uint8(0x81)) == 2
    assert e4m3.ulp_distance(np.uint8(0x38), np.uint8(0x39)) == 1


def _nearest_f32_is(s32: np.float32, exact: Fraction) -> bool:
    """s32 is the float32 nearest to the rational ``exact`` (no tie check needed here)."""
    up = np.nextafter(s32, np.float32(np.inf))
    dn = np.nextafter(s32, np.float32(-np.inf))
    d0 = abs(Fraction(float(s32)) - exact)
    return d0 <= abs(Fraction(float(up)) - exact) and d0 <= abs(Fraction(float(dn)) - exact)


def test_quantize_properties():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 128)) * rng.choice([1e-3, 1.0, 50.0], size=(64, 1))
    codes, scale = e4m3.quantize(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    for r in range(x.shape[0]):
        a = np.max(np.abs(x[r]))
        # scale is the float32 nearest to a/448
        assert _nearest_f32_is(scale[r], Fraction(float(a)) / 448)
        j = int(np.argmax(np.abs(x[r])))
        # the absmax element lands on +-448 (0x7E / 0xFE) up to the fp32 rounding of the scale
        assert e4m3.ulp_distance(codes[r, j], np.uint8(0x7E if x[r, j] > 0 else 0xFE)) <= 1
    deq = e4m3.dequantize(codes, scale)
    # each element is within half a code step of the exact value
    y = x / scale.astype(np.float64)[:, None]
    grid = e4m3.DECODE_TABLE[:127]
    idx = np.clip(np.searchsorted(grid, np.abs(y)), 1, 126)
    half_step = (grid[idx] - grid[idx - 1]) / 2
    assert np.all(np.abs(deq - x) <= half_step * scale.astype(np.float64)[:, None] * (1 + 1e-12))


def test_quantize_zero_vector():
    codes, scale = e4m3.quantize(np.zeros((3, 16)))
    assert np.all(codes == 0) and np.all(scale == 0)

"""FP8 e4m3fn codec and per-vector absmax quantisation (oracle, float64).

Test infrastructure only (see ``oracle/__init__.py``).

The pages say only that K and V are FP8-quantised once, at write time
(Runway Characters, abstract).  The format read here is the OCP 8-bit
floating-point e4m3 "fn" variant: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals m * 2^-9, largest finite magnitude 448, the two
codes 0x7F and 0xFF are NaN and there is no infinity.

Encoding saturates: magnitudes above 448 become 448.  Rounding is to the
nearest representable value, ties to the even code (the even mantissa).

Quantisation of one vector x (one token of one head):
    a     = max_i |x_i|
    scale = a / 448 rounded to float32  (the value the cache stores)
    code  = encode(x_i / scale), the division done in float64
    a = 0 gives scale = 0 and all codes 0.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_one(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: value of every code 0..255 (float64; NaN for 0x7F and 0xFF)
DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# Non-negative finite values, ascending; index == code for codes 0..126.
_POS_VALUES = DECODE_TABLE[:127].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8) -> float64 values."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """float64 -> e4m3fn codes (uint8): saturate to +-448, round to nearest,
    ties to the even code.  NaN encodes to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")  # first value >= mag
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - mag
    d_lo = mag - _POS_VALUES[lo]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def quantize(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Absmax quantisation along the last axis.

    Returns (codes uint8 with x's shape, scale float32 with x's shape minus
    the last axis)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1)
    scale = (a / E4M3_MAX).astype(np.float32)
    s64 = scale.astype(np.float64)[..., None]
    safe = np.where(s64 > 0, s64, 1.0)
    codes = encode(x / safe)
    codes = np.where(s64 > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes * scale in float64 (exact: 4 significant bits times 24)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in code steps between two code arrays.

    ord(c) = +-(c & 0x7F) by the sign bit, so +0 and -0 both map to 0 and
    the step across zero is counted once."""
    def _ord(c):
        c = np.asarray(c, dtype=np.int32)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    return np.abs(_ord(a) - _ord(b))

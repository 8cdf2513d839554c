"""8-bit E4M3 floating point codes for an FP8 KV cache — TEST INFRASTRUCTURE ONLY.

Format (OCP 8-bit floating point specification, E4M3 variant): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits.  Exponent field e > 0 gives
(1 + m/8) * 2^(e-7); e = 0 gives the subnormals m/8 * 2^-6 = m * 2^-9.
There are no infinities; S.1111.111 is NaN, so the largest finite magnitude
is 1.75 * 2^8 = 448 (code 0x7E).

The pages mention 8-bit floats only for model weights ("vLLM" documentation
page, tuning section).  Storing the KV cache as E4M3 codes with one scale
per KV head (a code c of head h stands for c * scale[h]) is this library's
extension; the reading is listed in the design doc.

Encoding a value x of KV head h: y = float32(x) / float32(scale[h]) in
float32 (IEEE division, correctly rounded), clamped to [-448, 448], then
rounded to the nearest code value, ties to the code with an even mantissa.
The nearest code is found by brute force over the table of all finite code
values, which is the definition written out.  Zero keeps its sign.  A NaN
stays NaN: it takes the NaN code S.1111.111 with the sign bit of x (the
format's only NaN encodings; infinities, which the format lacks, saturate
with every other magnitude beyond 448).
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


def value(code: int) -> float:
    """Exact value of a code (float64); NaN for the two NaN codes."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# finite non-negative codes 0x00..0x7E and their values, ascending
_CODES = np.arange(0x7F, dtype=np.int64)
_VALUES = np.array([value(c) for c in _CODES])
assert (np.diff(_VALUES) > 0).all()


def decode(codes) -> np.ndarray:
    """float64 values of an array of codes (uint8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, _VALUES[np.minimum(c & 0x7F, 0x7E)])
    return np.where(c & 0x80, -mag, mag)


def encode_f32(y) -> np.ndarray:
    """Codes (uint8) of float32 values y: clamp to +-448, round to nearest
    code value, ties to the even-mantissa code."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    sign = np.signbit(y)
    a = np.minimum(np.abs(y), MAX)
    nan = np.isnan(a)
    a = np.where(nan, MAX, a)  # placeholder magnitude; the NaN code is set below
    hi = np.searchsorted(_VALUES, a, side="left")  # first code value >= a
    hi = np.minimum(hi, len(_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _VALUES[lo]
    dhi = _VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_CODES[hi] % 2 == 0))
    code = np.where(a == _VALUES[hi], _CODES[hi], np.where(pick_hi, _CODES[hi], _CODES[lo]))
    code = np.where(nan, 0x7F, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize(x_f64, scale_f32) -> np.ndarray:
    """Codes of values x (exactly representable in float32, e.g. bf16 data)
    for a float32 scale: encode_f32(float32(x) / float32(scale))."""
    x32 = np.asarray(x_f64, dtype=np.float32)
    codes = encode_f32(x32 / np.float32(scale_f32))
    # a NaN's code carries the sign bit of x itself (the sign of a quotient
    # NaN is not fixed by IEEE arithmetic)
    return np.where(np.isnan(x32), np.where(np.signbit(x32), 0xFF, 0x7F), codes).astype(np.uint8)

"""Pins of the oracle's E4M3 codes (oracle/fp8.py) against the format's
definition and an independent implementation.

The format (OCP 8-bit floating point, E4M3): bias 7, no infinities, 448 the
largest finite magnitude, subnormals m * 2^-9.  Pins: code values that
follow from the bit layout by hand, every finite code encoding back to
itself, round-to-nearest ties to the even mantissa, saturation, and
agreement with torch's float8_e4m3fn conversion over random in-range data.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8


def test_code_values_from_the_bit_layout():
    assert fp8.value(0x38) == 1.0            # e = 7, m = 0
    assert fp8.value(0x3C) == 1.5            # m = 4
    assert fp8.value(0x7E) == 448.0          # e = 15, m = 6: 1.75 * 2^8
    assert fp8.value(0x77) == 240.0          # e = 14, m = 7: 1.875 * 2^7
    assert fp8.value(0x08) == 2.0 ** -6      # smallest normal
    assert fp8.value(0x01) == 2.0 ** -9      # smallest subnormal
    assert fp8.value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert fp8.value(0xB8) == -1.0
    assert fp8.value(0x00) == 0.0 and math.copysign(1, fp8.value(0x80)) == -1
    assert math.isnan(fp8.value(0x7F)) and math.isnan(fp8.value(0xFF))
    finite = [fp8.value(c) for c in range(256) if c & 0x7F != 0x7F]
    assert len(finite) == 254 and max(finite) == 448.0 and min(finite) == -448.0


def test_every_finite_code_encodes_back_to_itself():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = fp8.decode(codes)
    assert (fp8.encode_f32(vals.astype(np.float32)) == codes).all()


def test_round_to_nearest_ties_to_even():
    cases = {
        1.0625: 0x38,          # halfway 1.0 (m=0) / 1.125 (m=1): even m=0
        1.1875: 0x3A,          # halfway 1.125 / 1.25: even m=2
        1.07: 0x39,            # nearer 1.125
        2.0 ** -10: 0x00,      # halfway 0 / 2^-9: even code 0
        3 * 2.0 ** -10: 0x02,  # halfway 2^-9 (m=1) / 2^-8 (m=2): even m=2
        0.0175: 0x09,          # 1.12 * 2^-6: nearer 1.125 * 2^-6 (e=1, m=1)
        -3.3: 0xC5,            # nearer -3.25 (e=8, m=5)
    }
    for x, code in cases.items():
        assert int(fp8.encode_f32(np.float32(x))) == code, (x, hex(code))


def test_saturation_and_clamp():
    assert int(fp8.encode_f32(np.float32(448.0))) == 0x7E
    assert int(fp8.encode_f32(np.float32(464.0))) == 0x7E   # halfway to 480, still 448
    assert int(fp8.encode_f32(np.float32(500.0))) == 0x7E
    assert int(fp8.encode_f32(np.float32(-1e30))) == 0xFE
    assert int(fp8.encode_f32(np.float32(-0.0))) == 0x80


def test_nan_keeps_its_sign_and_agrees_with_torch():
    # the format's NaN encodings are S.1111.111; torch's float8_e4m3fn
    # conversion (an independent implementation) gives the same codes
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert list(fp8.encode_f32(x)) == [0x7F, 0xFF] == list(ref)
    assert list(fp8.quantize(x.astype(np.float64), np.float32(0.02))) == [0x7F, 0xFF]
    assert np.isnan(fp8.decode(np.array([0x7F, 0xFF], np.uint8))).all()
    # infinities saturate (the cache write clamps before converting)
    assert list(fp8.encode_f32(np.array([np.inf, -np.inf], np.float32))) == [0x7E, 0xFE]


def test_agrees_with_torch_float8_e4m3fn_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 60, 20000),
                        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (fp8.encode_f32(x) == ref).all()


def test_quantize_divides_by_the_scale_in_float32():
    scale = np.float32(0.0123)
    x = np.float32(1.7)
    assert int(fp8.quantize(np.float64(x), scale)) == int(fp8.encode_f32(x / scale))
    # the dequantised value is the code value times the scale
    code = fp8.quantize(np.float64(x), scale)
    assert abs(fp8.decode(code) * float(scale) - float(x)) <= 0.0625 * float(x)


@pytest.mark.parametrize("mistake", ["bias8", "truncate"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "bias8":
        def value8(code):
            code = int(code) & 0xFF
            e, m = (code >> 3) & 15, code & 7
            v = m * 2.0 ** -10 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8)
            return -v if code & 0x80 else v
        monkeypatch.setattr(fp8, "value", value8)
        with pytest.raises(AssertionError):
            test_code_values_from_the_bit_layout()
    else:
        def trunc(y):
            y = np.asarray(y, np.float32).astype(np.float64)
            a = np.minimum(np.abs(y), fp8.MAX)
            idx = np.searchsorted(fp8._VALUES, a, side="right") - 1
            return (fp8._CODES[idx] | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)
        monkeypatch.setattr(fp8, "encode_f32", trunc)
        with pytest.raises(AssertionError):
            test_round_to_nearest_ties_to_even()

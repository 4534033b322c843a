"""Pins for the oracle's E4M3FN decoding (closed forms + library cast)."""
import math

import numpy as np
import pytest
import torch

from oracle import E4M3FN_TABLE, decode_e4m3fn, e4m3fn_value


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0),
    (0x01, 2.0 ** -9),          # smallest subnormal
    (0x07, 7 * 2.0 ** -9),      # largest subnormal
    (0x08, 2.0 ** -6),          # smallest normal
    (0x38, 1.0),                # exponent field 7 = bias
    (0x40, 2.0),
    (0x3C, 1.5),
    (0x7E, 448.0),              # largest finite
    (0xB8, -1.0),
    (0xFE, -448.0),
])
def test_closed_form_values(code, value):
    assert e4m3fn_value(code) == value
    assert E4M3FN_TABLE[code] == value


def test_negative_zero_and_nans():
    assert E4M3FN_TABLE[0x80] == 0.0 and math.copysign(1.0, E4M3FN_TABLE[0x80]) == -1.0
    nan_codes = [c for c in range(256) if math.isnan(E4M3FN_TABLE[c])]
    assert nan_codes == [0x7F, 0xFF]


def test_matches_library_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(lib, E4M3FN_TABLE)  # NaNs compare equal here


def test_positive_codes_strictly_increase_and_mirror():
    pos = E4M3FN_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(E4M3FN_TABLE[0x80:0xFF], -pos)


def test_every_finite_value_is_exact_in_fp16():
    fin = E4M3FN_TABLE[np.isfinite(E4M3FN_TABLE)]
    np.testing.assert_array_equal(fin.astype(np.float16).astype(np.float64), fin)


def test_decode_requires_uint8():
    with pytest.raises(TypeError):
        decode_e4m3fn(np.array([1, 2], dtype=np.int32))
    np.testing.assert_array_equal(decode_e4m3fn(np.array([0x38, 0xC0], np.uint8)), [1.0, -2.0])

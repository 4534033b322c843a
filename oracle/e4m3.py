"""E4M3 value decoding from the bit fields.

[asym] section "What changes in vLLM's prefill routing?" stores values as
"FP8 E4M3"; the pages do not name the variant.  Reading taken: the OCP FP8
E4M3FN encoding (exponent bias 7, no infinities, NaN = S.1111.111), the only
E4M3 variant whose maximum finite value is 448, which the value scale
absmax/448 presumes.

Bit fields of a code b: sign s = b >> 7, exponent e = (b >> 3) & 15,
mantissa m = b & 7.
  e = 15 and m = 7  -> NaN
  e = 0             -> (-1)^s * m * 2^-9          (subnormal)
  otherwise         -> (-1)^s * (8 + m) * 2^(e - 10)
"""
import math

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one E4M3FN code, computed from its bits in float64."""
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code out of range")
    s = code >> 7
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (8 + m) * 2.0 ** (e - 10)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of uint8 E4M3FN codes."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return E4M3FN_TABLE[codes]

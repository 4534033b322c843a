"""Inputs that separate the scaled gather's rounding contract (fp32 product of the E4M3
value and the page scale, then RNE to fp16) from a single rounding of the exact product,
as a fused multiply-and-narrow instruction would do.

The two differ only on a few significand pairs: for E4M3 significand 1.5 (codes
with mantissa field 4) and fp32 scales in [1, 2), on 512 of the 2^23 scale
significands.  The pattern is invariant under powers of two while the fp16 result
stays normal, so every code 1.5 x 2^e with such a scale is a separating case.
"""
import functools

import numpy as np


@functools.lru_cache(maxsize=None)
def separating_scales() -> np.ndarray:
    """All fp32 s in [1, 2) with fp16(fp32(3 s)) != fp16(3 s) (numpy casts: the float32
    one rounds the exact float64 product, the float16 ones round to nearest even)."""
    sig = np.arange(1 << 23, 1 << 24, dtype=np.float64)
    exact = 3.0 * sig * 2.0 ** -23
    two_step = exact.astype(np.float32).astype(np.float16)
    one_step = exact.astype(np.float16)
    return (sig[two_step.view(np.uint16) != one_step.view(np.uint16)] * 2.0 ** -23).astype(np.float32)


def codes_with_significand_1_5(n: int, rng: np.random.Generator) -> np.ndarray:
    """n E4M3FN codes of value +-1.5 x 2^(e - 7), e in 1..15 (normal, finite)."""
    e = rng.integers(1, 16, size=n)
    sign = rng.integers(0, 2, size=n)
    return ((sign << 7) | (e << 3) | 4).astype(np.uint8)

"""Pins for the oracle's cache writer: the E4M3FN encoder and page compaction.

Pinned against closed forms worked by hand on the E4M3FN grid, brute force
over all 254 finite codes, the library cast torch.float8_e4m3fn (which does
not saturate, so it is compared inside [-448, 448]), and invariants of the
per-page-per-head absmax scale.
"""
import math

import numpy as np
import pytest
import torch

from oracle import E4M3FN_TABLE
from oracle.writer import (append_tokens, encode_e4m3fn, encode_e4m3fn_array, quantize_page,
                           quantize_pages)
from mixed_precision_paged_amd import synth

FINITE = [c for c in range(256) if not math.isnan(E4M3FN_TABLE[c])]


@pytest.mark.parametrize("x,code", [
    (0.0, 0x00), (-0.0, 0x80),
    (1.0, 0x38), (-1.0, 0xB8),
    (0.3, 0x2A),                 # binade [1/4, 1/2), step 1/32: 0.3 -> 10/32 = 0.3125
    (17.0, 0x58),                # tie 16 | 18 -> even mantissa (16)
    (19.0, 0x5A),                # tie 18 | 20 -> even mantissa (20)
    (2.0 ** -9, 0x01),           # smallest subnormal
    (2.0 ** -10, 0x00),          # tie 0 | 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),      # tie 1 | 2 (x 2^-9) -> 2
    (7.5 * 2.0 ** -9, 0x08),     # tie 7 | 8 (x 2^-9): even -> 2^-6, the smallest normal
    (447.0, 0x7E), (448.0, 0x7E),
    (464.0, 0x7E),               # tie 448 | 480 (480 is not finite): even mantissa 448
    (1000.0, 0x7E), (-1e30, 0xFE), (math.inf, 0x7E), (-math.inf, 0xFE),
    (math.nan, 0x7F), (-math.nan, 0x7F),
])
def test_closed_form_codes(x, code):
    assert encode_e4m3fn(x) == code
    assert int(encode_e4m3fn_array(np.array([x]))[0]) == code


def test_every_finite_code_round_trips():
    vals = np.array([E4M3FN_TABLE[c] for c in FINITE])
    assert [encode_e4m3fn(float(v)) for v in vals] == FINITE
    np.testing.assert_array_equal(encode_e4m3fn_array(vals), np.array(FINITE, np.uint8))


def _grid_probes():
    """All midpoints between neighbouring finite values, and one fp32 ulp either side."""
    pos = np.array(sorted(E4M3FN_TABLE[c] for c in FINITE if c < 0x80), np.float32)
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    x = np.concatenate([mids, up, dn, pos])
    return np.concatenate([x, -x])


def test_ties_go_to_even_mantissa():
    pos = sorted(E4M3FN_TABLE[c] for c in FINITE if c < 0x80)
    for lo, hi in zip(pos[:-1], pos[1:]):
        code = encode_e4m3fn((lo + hi) / 2)
        assert code & 1 == 0
        assert E4M3FN_TABLE[code] in (lo, hi)


def test_matches_library_cast_inside_the_range():
    rng = np.random.default_rng(7)
    fp16 = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float32)
    fp16 = fp16[np.isfinite(fp16) & (np.abs(fp16) <= 448)]
    rand = (rng.standard_normal(200_000) * rng.choice([1e-3, 0.1, 1, 30, 200], 200_000)).astype(np.float32)
    x = np.clip(np.concatenate([fp16, _grid_probes(), rand]), -448, 448).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(encode_e4m3fn_array(x), lib)


def test_nearest_by_brute_force():
    rng = np.random.default_rng(8)
    x = rng.uniform(-460, 460, 3000) * rng.choice([1, 1e-2, 1e-4], 3000)
    grid = np.array([E4M3FN_TABLE[c] for c in FINITE])
    codes = encode_e4m3fn_array(x)
    for xi, c in zip(x, codes):
        best = np.min(np.abs(grid - np.clip(xi, -448, 448)))
        assert abs(E4M3FN_TABLE[c] - np.clip(xi, -448, 448)) == best


def test_scalar_and_array_forms_agree():
    rng = np.random.default_rng(9)
    x = np.concatenate([_grid_probes(), rng.standard_normal(20000) * 50, [np.nan, np.inf, -np.inf]])
    np.testing.assert_array_equal(encode_e4m3fn_array(x),
                                  np.array([encode_e4m3fn(float(v)) for v in x], np.uint8))


# ---- page quantization -------------------------------------------------------------------------

def _page(rng, hkv=2, d=32, scale=1.0):
    k = rng.standard_normal((16, hkv, d)).astype(np.float16)
    v = (rng.standard_normal((16, hkv, d)) * scale).astype(np.float16)
    return k, v


def test_exact_page_reconstructs_exactly():
    """V already on the E4M3 grid times a power of two, with 448 present: scale = that power."""
    rng = np.random.default_rng(1)
    codes = rng.choice(FINITE, size=(16, 2, 32)).astype(np.uint8)
    codes[3, 0, 5] = 0x7E
    codes[9, 1, 0] = 0xFE
    s = np.array([2.0 ** -5, 2.0 ** -9], np.float32)
    v = (E4M3FN_TABLE[codes] * s[None, :, None]).astype(np.float16)
    assert np.array_equal(v.astype(np.float64), E4M3FN_TABLE[codes] * s[None, :, None])  # exact in fp16
    k = rng.standard_normal((16, 2, 32)).astype(np.float16)
    kk, c, sc = quantize_page(k, v)
    np.testing.assert_array_equal(sc, s)
    want = codes.copy()
    np.testing.assert_array_equal(c, want)
    np.testing.assert_array_equal(kk.view(np.uint16), k.view(np.uint16))


def test_scale_is_absmax_over_448_and_peak_saturates_to_448():
    rng = np.random.default_rng(2)
    for trial in range(20):
        k, v = _page(rng, scale=rng.choice([1e-3, 1.0, 40.0]))
        n = int(rng.integers(1, 17))
        _, c, s = quantize_page(k[:n], v[:n])
        for h in range(v.shape[1]):
            absmax = np.float32(np.abs(v[:n, h].astype(np.float32)).max())
            assert s[h] == np.float32(absmax / np.float32(448.0))
            assert np.max(c[:n, h] & 0x7F) == 0x7E


def test_dequantized_error_within_half_an_e4m3_step():
    rng = np.random.default_rng(3)
    k, v = _page(rng, hkv=4, d=64, scale=3.0)
    _, c, s = quantize_page(k, v)
    x = v.astype(np.float64) / s[None, :, None]
    back = E4M3FN_TABLE[c]
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(back - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4 * (1 + 1e-6))
    assert np.all(np.abs(back - x)[~normal] <= 2.0 ** -10 * (1 + 1e-6))


def test_partial_page_reads_n_rows_and_zeroes_the_rest():
    rng = np.random.default_rng(4)
    k, v = _page(rng)
    kk, c, s = quantize_page(k[:9], v[:9])
    assert np.all(kk[9:].view(np.uint16) == 0) and np.all(c[9:] == 0)
    np.testing.assert_array_equal(kk[:9].view(np.uint16), k[:9].view(np.uint16))
    _, c16, _ = quantize_page(k, v)
    full_max = np.abs(v.astype(np.float32)).max(axis=(0, 2))
    part_max = np.abs(v[:9].astype(np.float32)).max(axis=(0, 2))
    np.testing.assert_array_equal(s, (part_max / np.float32(448)).astype(np.float32))
    if np.any(full_max != part_max):   # rows 9..15 raise some head's absmax
        assert not np.array_equal(c16[:9], c[:9])


def test_empty_page_is_zero_with_unit_scale():
    kk, c, s = quantize_page(np.zeros((0, 3, 8), np.float16), np.zeros((0, 3, 8), np.float16))
    assert np.all(kk.view(np.uint16) == 0) and np.all(c == 0) and np.all(s == 1.0)


def test_pages_follow_row_starts():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((40, 2, 16)).astype(np.float16)
    v = rng.standard_normal((40, 2, 16)).astype(np.float16)
    starts, ns = [0, 16, 32, 5], [16, 16, 8, 3]
    K, C, S = quantize_pages(k, v, starts, ns)
    for i, (r, n) in enumerate(zip(starts, ns)):
        kk, c, s = quantize_page(k[r:r + n], v[r:r + n])
        np.testing.assert_array_equal(K[i].view(np.uint16), kk.view(np.uint16))
        np.testing.assert_array_equal(C[i], c)
        np.testing.assert_array_equal(S[i], s)


def test_zero_head_gets_unit_scale():
    rng = np.random.default_rng(5)
    k, v = _page(rng)
    v[:, 1] = np.float16(0.0)
    v[2, 1, 3] = np.float16(-0.0)
    _, c, s = quantize_page(k, v)
    assert s[1] == np.float32(1.0)
    assert np.all((c[:, 1] & 0x7F) == 0) and c[2, 1, 3] == 0x80


def test_agrees_with_library_quantizer_of_the_input_generator():
    """The generator's torch-based quantizer (clamp, float8 cast) gives the same codes and scales."""
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((5, 16, 2, 32)) * 7).astype(np.float16)
    k = rng.standard_normal((5, 16, 2, 32)).astype(np.float16)
    v[2] *= np.float16(1e-4)
    _, c, s = quantize_pages(k.reshape(80, 2, 32), v.reshape(80, 2, 32), np.arange(5) * 16, [16] * 5)
    lib_c, lib_s = synth.quantize_pages_e4m3(v, np.full(5, 16))
    np.testing.assert_array_equal(s, lib_s)
    np.testing.assert_array_equal(c, lib_c)


def test_append_writes_only_the_named_slots():
    rng = np.random.default_rng(10)
    kp = rng.standard_normal((6, 16, 2, 8)).astype(np.float16)
    vp = rng.standard_normal((6, 16, 2, 8)).astype(np.float16)
    kn = rng.standard_normal((3, 2, 8)).astype(np.float16)
    vn = rng.standard_normal((3, 2, 8)).astype(np.float16)
    pages, slots = np.array([4, 0, 4]), np.array([15, 0, 3])
    k2, v2 = append_tokens(kp, vp, kn, vn, pages, slots)
    touched = np.zeros((6, 16), bool)
    touched[pages, slots] = True
    np.testing.assert_array_equal(k2[~touched], kp[~touched])
    np.testing.assert_array_equal(v2[~touched], vp[~touched])
    for i in range(3):
        np.testing.assert_array_equal(k2[pages[i], slots[i]], kn[i])
        np.testing.assert_array_equal(v2[pages[i], slots[i]], vn[i])

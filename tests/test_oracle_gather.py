"""Pins for the oracle's compact-page gather (library float8/float32/float16 casts)."""
import numpy as np
import torch

import oracle
from mixed_precision_paged_amd import synth


def _case():
    return synth.make_paged_case(3, [37, 64, 16], 4, 2, 32, compact_frac=1.0)


def test_keys_are_bit_copies_in_page_id_order():
    c = _case()
    ids = np.array([5, 0, 3, 3], np.int32)
    ws_k, _ = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
    for i, p in enumerate(ids):
        np.testing.assert_array_equal(ws_k[i].view(np.uint16), c.k_compact[p].view(np.uint16))


def test_unscaled_values_match_library_cast():
    c = _case()
    ids = np.arange(c.k_compact.shape[0], dtype=np.int32)
    _, ws_v = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, False)
    lib = torch.from_numpy(c.v_compact).view(torch.float8_e4m3fn).to(torch.float16).numpy()
    np.testing.assert_array_equal(np.isnan(ws_v), np.isnan(lib))
    fin = ~np.isnan(lib)
    np.testing.assert_array_equal(ws_v.view(np.uint16)[fin], lib.view(np.uint16)[fin])


def test_scaled_values_match_library_fp32_multiply_then_fp16():
    c = _case()
    ids = np.array([2, 7, 1], np.int32)
    _, ws_v = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
    v = torch.from_numpy(c.v_compact[ids]).view(torch.float8_e4m3fn).to(torch.float32)
    s = torch.from_numpy(c.v_scale[ids])[:, None, :, None]
    lib = (v * s).to(torch.float16).numpy()
    fin = ~np.isnan(lib)
    np.testing.assert_array_equal(np.isnan(ws_v), ~fin)
    np.testing.assert_array_equal(ws_v.view(np.uint16)[fin], lib.view(np.uint16)[fin])


def test_nan_codes_become_nan():
    c = _case()
    v = c.v_compact.copy()
    v[0, 0, 0, :4] = [0x7F, 0xFF, 0x00, 0x80]
    _, ws_v = oracle.gather_compact_pages(c.k_compact, v, c.v_scale, [0], False)
    assert np.isnan(ws_v[0, 0, 0, 0]) and np.isnan(ws_v[0, 0, 0, 1])
    assert ws_v[0, 0, 0, 2] == 0 and ws_v[0, 0, 0, 3].view(np.uint16) == 0x8000


def test_scaled_values_round_the_fp32_product_not_the_exact_one():
    """The scaled gather multiplies in fp32 and then rounds to fp16.  On codes 1.5 x 2^e and
    scales where that differs from rounding the exact product once, the oracle must give
    the two-step result for every element."""
    from rounding_cases import codes_with_significand_1_5, separating_scales

    scales = separating_scales()
    assert scales.size == 512
    rng = np.random.default_rng(11)
    hkv, d = 8, 16
    pages = 8
    codes = codes_with_significand_1_5(pages * 16 * hkv * d, rng).reshape(pages, 16, hkv, d)
    v_scale = rng.choice(scales, size=(pages, hkv)).astype(np.float32)
    k = np.zeros((pages, 16, hkv, d), np.float16)
    _, ws_v = oracle.gather_compact_pages(k, codes, v_scale, np.arange(pages, dtype=np.int32), True)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    exact = vals * v_scale.astype(np.float64)[:, None, :, None]
    two_step = exact.astype(np.float32).astype(np.float16)
    one_step = exact.astype(np.float16)
    np.testing.assert_array_equal(ws_v.view(np.uint16), two_step.view(np.uint16))
    assert np.all(ws_v.view(np.uint16) != one_step.view(np.uint16))

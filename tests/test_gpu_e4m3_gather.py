"""GPU parity: device E4M3 decoding and the compact-page gather (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DeviceCase, dev, ekv, step
from mixed_precision_paged_amd import synth

pytestmark = pytest.mark.gpu


CODES = np.concatenate([np.roll(np.arange(256, dtype=np.uint8), k) for k in range(4)])  # every byte position


def _device_e4m3(method, scale_exp):
    codes = dev(CODES)
    out = torch.empty(CODES.size, dtype=torch.float16, device="cuda")
    ekv().ekv_e4m3_to_f16(codes, out, method, scale_exp)
    return out.cpu().numpy()


def _mismatches(got, scale_exp):
    """Codes whose device value differs from the oracle table times 2^scale_exp rounded to
    fp16 (nearest, ties to even; numpy's cast of the exact float64 product)."""
    want = (oracle.E4M3FN_TABLE[CODES] * 2.0 ** scale_exp).astype(np.float16)
    nan = np.isnan(want)
    assert np.all(np.isnan(got[nan]))
    return np.flatnonzero(got.view(np.uint16)[~nan] != want.view(np.uint16)[~nan])


@pytest.mark.parametrize("method", [0, 1])
def test_device_e4m3_matches_oracle_table(method):
    """Every code in every byte position of a packed word (codes run 0..255 four times,
    shifted by one each pass), unscaled and at the typical page scale 2^-7."""
    step(f"e4m3 table method {method}")
    for scale_exp in (0, -7):
        bad = _mismatches(_device_e4m3(method, scale_exp), scale_exp)
        assert bad.size == 0, (scale_exp, [int(CODES[i]) for i in bad[:8]])


def test_e4m3_expansion_over_every_page_scale_exponent():
    """Power-of-two scales 2^-33 .. 2^7 (page-head scales of fp16 values lie in that range:
    absmax / 448 with absmax from the smallest fp16 subnormal to 65504).  Both device paths --
    the gather's fp32 arithmetic and the conversion instruction the decode uses -- equal the
    oracle table times the scale rounded to fp16 (nearest, ties to even) at every exponent.
    Below 2^-15 that rounding is not the identity (code * 2^x leaves the fp16 grid), which is
    why the decode hands the instruction only -15..7 and applies the rest of the scale in fp32
    (its parity at such scales: test_compact_pages_with_extreme_page_scales)."""
    step("e4m3 expansion sweep over scale exponents -33..7")
    for method in (0, 1):
        for scale_exp in range(-33, 8):
            bad = _mismatches(_device_e4m3(method, scale_exp), scale_exp)
            assert bad.size == 0, (method, scale_exp, [int(CODES[i]) for i in bad[:8]])
    # the exact range: every code * 2^x is an fp16 value iff x in -15..7
    exact = [k for k in range(-33, 8)
             if np.array_equal((oracle.E4M3FN_TABLE[CODES] * 2.0 ** k).astype(np.float16).astype(np.float64),
                               oracle.E4M3FN_TABLE[CODES] * 2.0 ** k, equal_nan=True)]
    assert exact == list(range(-15, 8)), exact


def _gather_gpu(dc, ids, apply_scale, capacity=None):
    c = dc.case
    n = len(ids)
    cap = n if capacity is None else capacity
    ws_k = torch.full((cap, 16, c.num_kv_heads, c.head_dim), 7.0, dtype=torch.float16, device="cuda")
    ws_v = torch.full_like(ws_k, 7.0)
    ekv().ekv_gather_compact_pages(dc.kv(), dev(np.asarray(ids, np.int32)), apply_scale, ws_k, ws_v)
    torch.cuda.synchronize()
    return ws_k.cpu().numpy(), ws_v.cpu().numpy()


def _assert_bits(got, want):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got.view(np.uint16)[~nan], want.view(np.uint16)[~nan])


@pytest.mark.parametrize("apply_scale", [False, True])
def test_gather_tiny_pool_all_pages(apply_scale):
    step(f"gather tiny apply_scale={apply_scale}")
    c = synth.tiny_decode_case()
    dc = DeviceCase(c)
    ids = np.arange(16, dtype=np.int32)  # every pool page, including NaN-poisoned ones
    gk, gv = _gather_gpu(dc, ids, apply_scale)
    ok, ov = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, apply_scale)
    _assert_bits(gk, ok)
    _assert_bits(gv, ov)


@pytest.mark.parametrize("hkv,d", [(8, 128), (2, 64), (1, 128)])
@pytest.mark.parametrize("apply_scale", [False, True])
def test_gather_ragged_pages_with_repeats(hkv, d, apply_scale):
    step(f"gather ragged hkv={hkv} d={d} scale={apply_scale}")
    c = synth.make_paged_case(41, [37, 300, 1001, 16], 4 * hkv, hkv, d, compact_frac=1.0)
    dc = DeviceCase(c)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, c.k_compact.shape[0], size=97).astype(np.int32)
    ids[:3] = ids[3]  # repeated page ids are legal
    gk, gv = _gather_gpu(dc, ids, apply_scale, capacity=128)
    ok, ov = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, apply_scale)
    _assert_bits(gk[:97], ok)
    _assert_bits(gv[:97], ov)
    assert np.all(gk[97:] == 7.0) and np.all(gv[97:] == 7.0)  # capacity tail untouched


def test_gather_rejects_overflow_and_marks_bad_ids():
    step("gather errors")
    c = synth.make_paged_case(42, [64], 8, 2, 64, compact_frac=1.0)
    dc = DeviceCase(c)
    ws = torch.zeros((2, 16, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ekv().EkvError) as e:
        ekv().ekv_gather_compact_pages(dc.kv(), dev(np.zeros(3, np.int32)), True, ws, ws.clone())
    assert e.value.status == ekv().EKV_ERR_WORKSPACE_TOO_SMALL
    ids = np.array([0, c.k_compact.shape[0] + 5], np.int32)
    gk, gv = _gather_gpu(dc, ids, True)
    assert np.all(np.isnan(gk[1])) and np.all(np.isnan(gv[1]))
    ok, ov = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids[:1], True)
    _assert_bits(gk[:1], ok)
    _assert_bits(gv[:1], ov)


def test_scaled_gather_rounds_the_fp32_product_on_separating_scales():
    """Every value of these pages is a case where rounding the exact product once (a fused
    multiply-and-narrow) gives other bits than the fp32 product rounded to fp16."""
    from rounding_cases import codes_with_significand_1_5, separating_scales

    step("gather on scales that separate fp32-then-fp16 from one rounding")
    c = synth.make_paged_case(43, [16 * 12], 32, 8, 128, compact_frac=1.0)
    rng = np.random.default_rng(12)
    c.v_compact[:] = codes_with_significand_1_5(c.v_compact.size, rng).reshape(c.v_compact.shape)
    c.v_scale[:] = rng.choice(separating_scales(), size=c.v_scale.shape)
    dc = DeviceCase(c)
    ids = np.arange(c.v_compact.shape[0], dtype=np.int32)
    _, gv = _gather_gpu(dc, ids, True)
    _, ov = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
    _assert_bits(gv, ov)
    one_step = (oracle.E4M3FN_TABLE[c.v_compact] * c.v_scale.astype(np.float64)[:, None, :, None]).astype(np.float16)
    assert np.all(gv.view(np.uint16) != one_step.view(np.uint16))

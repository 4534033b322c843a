"""GPU parity: direct paged prefill (no workspace) against the oracle, and bit-equality
with the gather route (gather -> workspace prefill) on compact prompts."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, DeviceCase, assert_close, assert_lse_close, dev, ekv, f16_bits_equal_rne,
                         step)
from mixed_precision_paged_amd import synth

pytestmark = pytest.mark.gpu


def _paged(case, cu, max_len, out_dtype=torch.float32, causal=True, flags=True, pt=None):
    dc = DeviceCase(case)
    T = int(cu[-1])
    out = torch.full((T, case.num_q_heads, case.head_dim), 5.0, dtype=out_dtype, device="cuda")
    lse = torch.empty((T, case.num_q_heads), dtype=torch.float32, device="cuda")
    table = dc.page_table if pt is None else dev(pt)
    ekv().ekv_prefill_paged_attention(dc.kv(), dc.q, dev(np.asarray(cu, np.int32)), table,
                                      dc.fidelity if flags else None, max_len, case.sm_scale, out, lse,
                                      causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(case, cu, causal=True, rows=None, pt=None):
    return oracle.paged_prefill_attention(case.q, case.k_target, case.v_target, case.k_compact,
                                          case.v_compact, case.v_scale,
                                          case.page_table if pt is None else pt, case.fidelity, cu,
                                          causal, case.sm_scale, rows=rows)


def _gather_route(pc):
    """The gather route on the same prompts, all in one workspace."""
    c = pc.paged
    dc = DeviceCase(c)
    prompts = list(range(len(pc.prompt_lens)))
    ids, kv_start = pc.chunk_pages(prompts)
    ws_k = torch.empty((len(ids), 16, c.num_kv_heads, c.head_dim), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    ekv().ekv_gather_compact_pages(dc.kv(), dev(ids), True, ws_k, ws_v)
    out = torch.empty((c.q.shape[0], c.num_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.q.shape[0], c.num_q_heads), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_attention(dc.q, ws_k, ws_v, dev(pc.cu_seqlens_q), dev(kv_start),
                                int(pc.prompt_lens.max()), c.sm_scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 2, 64), (8, 8, 128), (16, 2, 64), (16, 8, 128), (4, 2, 64),
                                      (32, 4, 128)])
def test_compact_prompts_bit_equal_to_gather_route_and_match_oracle(hq, hkv, d):
    step(f"paged prefill compact hq={hq} hkv={hkv} d={d}")
    lens = [1, 17, 100, 257, 64, 130]
    pc = synth.make_prefill_case(400 + d + hq, lens, hq, hkv, d)
    c = pc.paged
    out, lse = _paged(c, pc.cu_seqlens_q, max(lens))
    g_out, g_lse = _gather_route(pc)
    assert np.array_equal(out.view(np.uint32), g_out.view(np.uint32)), "differs from the gather route"
    assert np.array_equal(lse.view(np.uint32), g_lse.view(np.uint32))
    want, wlse = _oracle(c, pc.cu_seqlens_q)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


@pytest.mark.parametrize("hq,hkv,d,causal", [(32, 8, 128, True), (8, 2, 64, True), (4, 1, 128, False),
                                             (16, 2, 128, False)])
def test_mixed_fidelity_prompts_match_oracle(hq, hkv, d, causal):
    step(f"paged prefill mixed fidelity hq={hq} hkv={hkv} d={d} causal={causal}")
    lens = [300, 1, 47, 128, 513]
    case = synth.make_paged_case(410 + d, lens, hq, hkv, d, compact_frac=0.5,
                                 query_rows=int(sum(lens)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out, lse = _paged(case, cu, max(lens), causal=causal)
    want, wlse = _oracle(case, cu, causal=causal)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


def test_mixed_fidelity_with_value_outliers():
    """1% of V elements x20: P is rounded to fp16 for the MFMA (as on the gather route), so
    the error bound scales with max|V| / 4 (4 ~ the page absmax of N(0,1) values)."""
    step("paged prefill mixed fidelity with x20 value outliers")
    lens = [300, 1, 47, 128, 513]
    case = synth.make_paged_case(415, lens, 32, 8, 128, compact_frac=0.5, outlier_frac=0.01,
                                 outlier_mult=20.0, query_rows=int(sum(lens)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out, lse = _paged(case, cu, max(lens))
    want, wlse = _oracle(case, cu)
    vmax = max(float(np.nanmax(np.abs(case.v_target.astype(np.float32)))),
               float(np.nanmax(case.v_scale)) * 448.0, 4.0)
    assert_close(out, want, tol=TOL * vmax / 4.0)
    assert_lse_close(lse, wlse)


def test_fp16_output_and_single_pool_without_flags():
    step("paged prefill fp16 out, flags NULL")
    pc = synth.make_prefill_case(420, [200, 77], 32, 8, 128)
    c = pc.paged
    o32, _ = _paged(c, pc.cu_seqlens_q, 200)
    o16, _ = _paged(c, pc.cu_seqlens_q, 200, out_dtype=torch.float16)
    assert f16_bits_equal_rne(o16, o32)
    onf, _ = _paged(c, pc.cu_seqlens_q, 200, flags=False)
    assert np.array_equal(onf.view(np.uint32), o32.view(np.uint32))


def test_bad_page_id_marks_its_row_tiles_nan():
    """An out-of-pool page id poisons the rows of every workgroup that stages its key tile.
    Below 2,048 tokens, with 4 query heads per KV head, a workgroup holds 32 positions of 4
    heads, so exactly the rows from the start of the bad page's 64-key tile are NaN."""
    step("paged prefill bad page id")
    lens = [400, 60]
    pc = synth.make_prefill_case(430, lens, 8, 2, 128)
    c = pc.paged
    pt = c.page_table.copy()
    pt[0, 10] = c.k_compact.shape[0] + 5          # keys 160..175 of prompt 0: row tiles 1.. read it
    out, lse = _paged(c, pc.cu_seqlens_q, max(lens), pt=pt)
    assert np.all(np.isnan(out[128:400])) and np.all(np.isnan(lse[128:400]))
    assert np.all(np.isfinite(out[:128])) and np.all(np.isfinite(out[400:]))
    want, wlse = _oracle(c, pc.cu_seqlens_q, rows=np.r_[0:128, 400:460])
    assert_close(out[:128], want[:128])
    assert_close(out[400:], want[400:])


def test_long_ragged_compact_prompts_bit_equal_to_gather_route():
    """From 2,048 tokens both routes run 256-row workgroups (the direct route stages half a
    page of each key tile per wavefront); ragged lengths leave partial pages, key tiles and
    row tiles at the ends, and the 1- and 17-token prompts share the launch."""
    step("paged prefill long ragged compact prompts (256-row workgroups)")
    lens = [2100, 1, 700, 2048, 17, 2305]
    pc = synth.make_prefill_case(440, lens, 8, 2, 128)
    c = pc.paged
    out, lse = _paged(c, pc.cu_seqlens_q, max(lens))
    g_out, g_lse = _gather_route(pc)
    assert np.array_equal(out.view(np.uint32), g_out.view(np.uint32)), "differs from the gather route"
    assert np.array_equal(lse.view(np.uint32), g_lse.view(np.uint32))
    want, wlse = _oracle(c, pc.cu_seqlens_q)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


@pytest.mark.parametrize("causal", [True, False])
def test_long_ragged_mixed_fidelity_prompts_match_oracle(causal):
    step(f"paged prefill long ragged mixed fidelity causal={causal}")
    lens = [2305, 1, 2048, 999]
    case = synth.make_paged_case(450, lens, 8, 2, 128, compact_frac=0.5, query_rows=int(sum(lens)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out, lse = _paged(case, cu, max(lens), causal=causal)
    want, wlse = _oracle(case, cu, causal=causal)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


def test_bad_page_id_in_a_long_prompt_marks_its_256_row_tiles_nan():
    """From 2,048 tokens a workgroup holds 256 positions of one head: rows 640.. read the bad
    page's tile, so the workgroup of rows 512..767 and every later one is NaN; every earlier
    row is computed and matches the oracle."""
    step("paged prefill bad page id, 256-row workgroups")
    lens = [2100, 60]
    pc = synth.make_prefill_case(460, lens, 8, 2, 128)
    c = pc.paged
    pt = c.page_table.copy()
    pt[0, 40] = c.k_compact.shape[0] + 5          # keys 640..655 of prompt 0: rows 640.. read it
    out, lse = _paged(c, pc.cu_seqlens_q, max(lens), pt=pt)
    assert np.all(np.isnan(out[512:2100])) and np.all(np.isnan(lse[512:2100]))
    assert np.all(np.isfinite(out[:512])) and np.all(np.isfinite(out[2100:]))
    want, wlse = _oracle(c, pc.cu_seqlens_q, rows=np.r_[0:512, 2100:2160])
    assert_close(out[:512], want[:512])
    assert_close(out[2100:], want[2100:])


@pytest.mark.parametrize("route", ["paged", "gather"])
def test_long_ragged_fp16_rows_are_rne_of_fp32_and_spare_rows_untouched(route):
    """From 2,048 tokens the fp16 output rows leave through LDS four whole rows per store: each
    must equal the RNE of the fp32 row, and query rows past the last prompt (present in q and
    out but in no prompt) must keep what they held, LSE included."""
    step(f"prefill fp16 rows through LDS, 256-row workgroups, {route} route")
    lens = [2100, 1, 700, 2305]
    pc = synth.make_prefill_case(470, lens, 8, 2, 128)
    c = pc.paged
    dc = DeviceCase(c)
    T, spare = int(pc.cu_seqlens_q[-1]), 40
    q = torch.cat([dc.q, torch.randn((spare, c.num_q_heads, c.head_dim), device="cuda").half()])
    cu = dev(pc.cu_seqlens_q)
    if route == "gather":
        ids, kv_start = pc.chunk_pages(list(range(len(lens))))
        ws_k = torch.empty((len(ids), 16, c.num_kv_heads, c.head_dim), dtype=torch.float16, device="cuda")
        ws_v = torch.empty_like(ws_k)
        ekv().ekv_gather_compact_pages(dc.kv(), dev(ids), True, ws_k, ws_v)
    outs = {}
    for dtype in (torch.float32, torch.float16):
        out = torch.full((T + spare, c.num_q_heads, c.head_dim), 7.0, dtype=dtype, device="cuda")
        lse = torch.full((T + spare, c.num_q_heads), 7.0, dtype=torch.float32, device="cuda")
        if route == "paged":
            ekv().ekv_prefill_paged_attention(dc.kv(), q, cu, dc.page_table, dc.fidelity, max(lens),
                                              c.sm_scale, out, lse)
        else:
            ekv().ekv_prefill_attention(q, ws_k, ws_v, cu, dev(kv_start), max(lens), c.sm_scale, out, lse)
        torch.cuda.synchronize()
        outs[dtype] = (out.cpu().numpy(), lse.cpu().numpy())
    (o32, l32), (o16, l16) = outs[torch.float32], outs[torch.float16]
    assert f16_bits_equal_rne(o16[:T], o32[:T])
    assert np.array_equal(l16[:T].view(np.uint32), l32[:T].view(np.uint32))
    assert np.all(o16[T:] == 7.0) and np.all(o32[T:] == 7.0)
    assert np.all(l16[T:] == 7.0) and np.all(l32[T:] == 7.0)
    want, wlse = _oracle(c, pc.cu_seqlens_q, rows=np.r_[0:64, 2036:2164, T - 300:T])
    sel = np.r_[0:64, 2036:2164, T - 300:T]
    assert_close(o32[sel], want[sel])
    assert_lse_close(l32[sel], wlse[sel])


def test_direct_route_expands_separating_scales_like_the_gather():
    """Compact pages whose every value separates the gather's fp32-then-fp16 rounding from a
    single rounding: the direct route must still match the gather route bit for bit."""
    from rounding_cases import codes_with_significand_1_5, separating_scales

    step("paged prefill on scales that separate the two roundings")
    lens = [300, 2100]
    pc = synth.make_prefill_case(480, lens, 8, 2, 128)
    c = pc.paged
    rng = np.random.default_rng(13)
    c.v_compact[:] = codes_with_significand_1_5(c.v_compact.size, rng).reshape(c.v_compact.shape)
    c.v_scale[:] = rng.choice(separating_scales(), size=c.v_scale.shape) * np.float32(2.0 ** -6)
    out, lse = _paged(c, pc.cu_seqlens_q, max(lens))
    g_out, g_lse = _gather_route(pc)
    assert np.array_equal(out.view(np.uint32), g_out.view(np.uint32)), "differs from the gather route"
    assert np.array_equal(lse.view(np.uint32), g_lse.view(np.uint32))

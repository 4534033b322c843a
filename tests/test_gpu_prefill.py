"""GPU parity: compact-prefill route (gather -> causal FP16 MFMA prefill) vs the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, DeviceCase, assert_close, assert_lse_close, dev, ekv,
                         f16_bits_equal_rne, max_abs, oracle_decode, step)
from mixed_precision_paged_amd import synth

pytestmark = pytest.mark.gpu


def _v_ratio(ws_v):
    """|V| of a workspace relative to N(0,1) data (whose page absmax is about 4)."""
    v = np.asarray(ws_v, dtype=np.float64)
    return max(1.0, float(np.nanmax(np.abs(v))) / 4.0)


def _route(pc, prompts, apply_scale=True, out_dtype=torch.float32, causal=True, capacity=None):
    """GPU: gather the prompts' pages, then prefill.  Returns (out, lse, ws_k, ws_v) on host."""
    c = pc.paged
    dc = DeviceCase(c)
    ids, kv_start = pc.chunk_pages(prompts)
    cap = len(ids) if capacity is None else capacity
    ws_k = torch.empty((cap, 16, c.num_kv_heads, c.head_dim), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    ekv().ekv_gather_compact_pages(dc.kv(), dev(ids), apply_scale, ws_k, ws_v)
    rows = np.concatenate([np.arange(pc.cu_seqlens_q[p], pc.cu_seqlens_q[p + 1]) for p in prompts])
    q = dev(c.q[rows])
    lens = pc.prompt_lens[list(prompts)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = torch.full((len(rows), c.num_q_heads, c.head_dim), 5.0, dtype=out_dtype, device="cuda")
    lse = torch.empty((len(rows), c.num_q_heads), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_attention(q, ws_k, ws_v, dev(cu), dev(kv_start), int(lens.max()), c.sm_scale,
                                out, lse, causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), ws_k.cpu().numpy(), ws_v.cpu().numpy(), rows, cu, kv_start


def _oracle_route(pc, prompts, rows, cu, kv_start, apply_scale=True, causal=True, sample=None):
    c = pc.paged
    ids, _ = pc.chunk_pages(prompts)
    wk, wv = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, apply_scale)
    wk = wk.reshape(-1, c.num_kv_heads, c.head_dim)
    wv = wv.reshape(-1, c.num_kv_heads, c.head_dim)
    return oracle.prefill_attention(c.q[rows], wk, wv, cu, kv_start, causal, c.sm_scale, rows=sample)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 64), (8, 2, 128), (16, 2, 64), (16, 8, 128), (4, 2, 64),
                                      (16, 2, 128)])
def test_prefill_route_ragged_prompts(hq, hkv, d):
    """Ragged prompts, every GQA group size: below 2,048 tokens a head-dim-128 workgroup
    takes 1, 2 or 4 query heads of one KV head (8 per KV head: two such groups)."""
    step(f"prefill ragged hq={hq} hkv={hkv} d={d}")
    lens = [1, 17, 100, 257, 64, 130]
    pc = synth.make_prefill_case(200 + d + hq, lens, hq, hkv, d)
    prompts = list(range(len(lens)))
    out, lse, *_, rows, cu, ks = _route(pc, prompts)
    want, wlse = _oracle_route(pc, prompts, rows, cu, ks)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


def test_prefill_fp16_output_is_rne_of_fp32_and_noncausal():
    step("prefill fp16 + noncausal")
    pc = synth.make_prefill_case(301, [200, 77], 32, 8, 128)
    out32, *_ = _route(pc, [0, 1])
    out16, *_ = _route(pc, [0, 1], out_dtype=torch.float16)
    assert f16_bits_equal_rne(out16, out32)
    out, lse, *_, rows, cu, ks = _route(pc, [0, 1], causal=False)
    want, wlse = _oracle_route(pc, [0, 1], rows, cu, ks, causal=False)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


def test_prefill_unscaled_gather_route():
    step("prefill unscaled route")
    pc = synth.make_prefill_case(302, [150, 33], 8, 2, 128)
    out, lse, wk, wv, rows, cu, ks = _route(pc, [1, 0], apply_scale=False)
    want, wlse = _oracle_route(pc, [1, 0], rows, cu, ks, apply_scale=False)
    # unscaled values are E4M3 codes (|v| up to 448, not N(0,1)): the bound scales with |V|
    assert_close(out, want, tol=TOL * _v_ratio(wv))
    assert_lse_close(lse, wlse)


def test_prefill_over_arbitrary_workspace_rows():
    """Prompts placed at gaps of NaN rows in K/V: only their own rows may be read."""
    step("prefill arbitrary rows")
    rng = np.random.default_rng(3)
    hq, hkv, d = 16, 4, 128
    lens = [5, 129, 300]
    starts, r = [], 0
    for n in lens:
        r += 7
        starts.append(r)
        r += n
    k = np.full((r + 9, hkv, d), np.nan, np.float16)
    v = np.full((r + 9, hkv, d), np.nan, np.float16)
    for s, n in zip(starts, lens):
        k[s:s + n] = rng.standard_normal((n, hkv, d))
        v[s:s + n] = rng.standard_normal((n, hkv, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((cu[-1], hq, d)).astype(np.float16)
    out = torch.empty((cu[-1], hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((cu[-1], hq), dtype=torch.float32, device="cuda")
    sm = 1 / np.sqrt(d)
    ekv().ekv_prefill_attention(dev(q), dev(k), dev(v), dev(cu), dev(np.array(starts, np.int32)),
                                max(lens), sm, out, lse)
    torch.cuda.synchronize()
    want, wlse = oracle.prefill_attention(q, k, v, cu, starts, True, sm)
    assert_close(out.cpu().numpy(), want)
    assert_lse_close(lse.cpu().numpy(), wlse)


def test_prefill_bad_offsets_give_nan_rows_not_faults():
    step("prefill bad offsets")
    hq, hkv, d = 8, 2, 64
    rng = np.random.default_rng(4)
    k = rng.standard_normal((100, hkv, d)).astype(np.float16)
    q = rng.standard_normal((60, hq, d)).astype(np.float16)
    cu = np.array([0, 30, 60], np.int32)
    starts = np.array([0, 90], np.int32)  # second prompt would read rows 90..119 of 100
    out = torch.zeros((60, hq, d), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_attention(dev(q), dev(k), dev(k), dev(cu), dev(starts), 30, 0.125, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o[:30])) and np.all(np.isnan(o[30:]))


def test_prefill_row_equals_decode_over_prefix():
    """Cross-kernel: prefill row i over a prompt == decode over its first i+1 tokens."""
    step("prefill vs decode prefix")
    pc = synth.make_prefill_case(303, [77], 32, 8, 128)
    pc.paged.v_scale[:] = 1.0  # unit scales: the unscaled workspace holds the decode values
    out, lse, wk, wv, *_ = _route(pc, [0], apply_scale=False)
    tol = 2 * TOL * _v_ratio(wv)  # unit scales: |V| up to 448
    dc = DeviceCase(pc.paged)
    for i in (0, 15, 16, 63, 76):
        q = dev(pc.paged.q[i:i + 1])
        lens = dev(np.array([i + 1], np.int32))
        od, ld = dc.decode(torch.float32, q=q, rows=[0], seq_lens=lens, max_seq_len=77)
        assert max_abs(out[i], od[0]) <= tol
        assert abs(float(lse[i, 0]) - float(ld[0, 0])) <= 2 * TOL


@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (64, 16, 2)])
def test_repeat_launches_give_identical_bits(d, hq, hkv):
    """Both prefill kernels, both sources (workspace and pages), launched repeatedly on the
    same inputs give the same bits: every LDS tile reuse is ordered by a barrier (including
    the first, where tile 2's keys land in the buffer tile 0's keys were read from)."""
    step(f"prefill repeat launches d={d}")
    pc = synth.make_prefill_case(91 + d, [700, 1029, 64, 333], hq, hkv, d)
    c = pc.paged
    dc = DeviceCase(c)
    prompts = list(range(len(pc.prompt_lens)))
    ids, kv_start = pc.chunk_pages(prompts)
    ws_k = torch.empty((len(ids), 16, hkv, d), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    ekv().ekv_gather_compact_pages(dc.kv(), dev(ids), True, ws_k, ws_v)
    q = dev(c.q)
    cu = dev(pc.cu_seqlens_q)
    L = int(pc.prompt_lens.max())
    first = {}
    for rep in range(6):
        for route in ("ws", "paged"):
            out = torch.empty((q.shape[0], hq, d), dtype=torch.float32, device="cuda")
            if route == "ws":
                ekv().ekv_prefill_attention(q, ws_k, ws_v, cu, dev(kv_start), L, c.sm_scale, out)
            else:
                ekv().ekv_prefill_paged_attention(dc.kv(), q, cu, dc.page_table, None, L, c.sm_scale, out)
            torch.cuda.synchronize()
            if rep == 0:
                first[route] = out
            else:
                assert torch.equal(out.view(torch.int32), first[route].view(torch.int32)), (route, rep)
    assert torch.equal(first["ws"].view(torch.int32), first["paged"].view(torch.int32))


def _rising_scores(lens, hq, hkv, d, seed):
    """Q, K, V (fp16) whose scores climb about 0.3 log2 units per key for the query rows whose
    first component is +4 and fall as fast for those with -4 (alternating every three rows), on
    top of N(0,1) noise: the running max of a climbing row moves past tau in nearly every 32-key
    unit, that of a falling row never after its first, and every wavefront holds both kinds."""
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    c = (1.0 / np.sqrt(d)) * np.log2(np.e)
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    off = 0
    for L in lens:
        j = np.arange(L)
        k[off:off + L, :, 0] = (0.3 * j / (4.0 * c))[:, None]
        q[off:off + L, :, 0] = np.where((j // 3) % 2 == 0, 4.0, -4.0)[:, None]
        off += L
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("lens,hq,hkv,d", [([2305, 700], 32, 8, 128), ([700, 130, 33], 32, 8, 128),
                                           ([1000, 77], 8, 2, 64)])
def test_prefill_running_max_moving_in_most_units(lens, hq, hkv, d):
    """Online softmax whose running max moves in most units (the rescale branch) for some rows of
    each wavefront and never for others: both routes against the oracle, and the direct route over
    TARGET pages bit-equal to the workspace route."""
    step(f"prefill rising scores lens={lens} hq={hq} hkv={hkv} d={d}")
    q, k, v = _rising_scores(lens, hq, hkv, d, 900 + d + len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ks = cu[:-1].copy()
    sm = 1.0 / np.sqrt(d)
    T = q.shape[0]
    out = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_attention(dev(q), dev(k), dev(v), dev(cu), dev(ks), int(max(lens)), sm, out, lse)
    _check_both_routes(q, k, v, lens, cu, ks, hkv, d, sm, out, lse)


def _check_both_routes(q, k, v, lens, cu, ks, hkv, d, sm, out, lse):
    """The direct route over the same rows as TARGET pages (prompt p's rows in its own pages, a
    permuted page order) bit-equal to the workspace route's out/lse, and sampled rows of both
    against the oracle."""
    npg = [(L + 15) // 16 for L in lens]
    pool_k = np.zeros((sum(npg), 16, hkv, d), np.float16)
    pool_v = np.zeros_like(pool_k)
    perm = np.random.default_rng(7).permutation(sum(npg)).astype(np.int32)
    pt = np.zeros((len(lens), max(npg)), np.int32)
    used = 0
    for p, L in enumerate(lens):
        for j in range(npg[p]):
            r0, r1 = int(cu[p]) + 16 * j, min(int(cu[p]) + 16 * j + 16, int(cu[p + 1]))
            pool_k[perm[used + j], :r1 - r0] = k[r0:r1]
            pool_v[perm[used + j], :r1 - r0] = v[r0:r1]
            pt[p, j] = perm[used + j]
        used += npg[p]
    kv = ekv().paged_kv(hkv, d, dev(pool_k), dev(pool_v))
    pout = torch.empty_like(out)
    plse = torch.empty_like(lse)
    ekv().ekv_prefill_paged_attention(kv, dev(q), dev(cu), dev(pt), None, int(max(lens)), sm, pout, plse)
    torch.cuda.synchronize()
    got, glse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(pout.cpu().numpy().view(np.uint32), got.view(np.uint32))
    assert np.array_equal(plse.cpu().numpy().view(np.uint32), glse.view(np.uint32))
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([rng.choice(np.arange(int(cu[p]), int(cu[p + 1])),
                                                  size=min(160, int(lens[p])), replace=False)
                                       for p in range(len(lens))]))
    want, wlse = oracle.prefill_attention(q, k, v, cu, ks, True, sm, rows=sample)
    assert_close(got[sample], want[sample])
    assert_lse_close(glse[sample], wlse[sample])


@pytest.mark.parametrize("lens,mult", [([2305, 700, 64], 3.0), ([700, 130, 33], 5.0), ([2100, 999], 5.0)])
def test_prefill_sharp_softmax_on_normal_data(lens, mult):
    """Softmax scale mult / sqrt(d) on N(0,1) data: each unit's scores spread over tens of log2
    units, so a row's first units are overtaken by far larger scores again and again and the
    redo of a unit whose weights pass 2^tau runs in many wavefronts.  Both routes against the
    oracle, the direct route over TARGET pages bit-equal to the workspace route."""
    step(f"prefill sharp softmax lens={lens} scale x{mult}")
    hq, hkv, d = 32, 8, 128
    rng = np.random.default_rng(950 + len(lens) + int(mult))
    T = int(sum(lens))
    q, k, v = (rng.standard_normal((T, h, d)).astype(np.float16) for h in (hq, hkv, hkv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ks = cu[:-1].copy()
    sm = mult / np.sqrt(d)
    out = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_attention(dev(q), dev(k), dev(v), dev(cu), dev(ks), int(max(lens)), sm, out, lse)
    _check_both_routes(q, k, v, lens, cu, ks, hkv, d, sm, out, lse)

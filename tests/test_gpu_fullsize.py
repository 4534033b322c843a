"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Decode: every output element against the oracle.  Gather: bit-exact on a full
4,096-page chunk.  Prefill: sampled rows (tile boundaries, first/last rows,
random rows) per prompt, every head, against the oracle row by row.  Mixed
batch: all 36 layers routed through one shared workspace, decode scratch and
output tensor, each layer's workspace bit-exact, decode rows fully checked,
prefill rows sampled, and every row written by exactly its own path.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DeviceCase, assert_close, assert_lse_close, dev, ekv, max_abs,
                         oracle_decode, step)
from mixed_precision_paged_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SAMPLE_ROWS = (0, 1, 15, 16, 63, 64, 127, 128, 129, 2047, 4095, 4096, 8190, 8191)


def _decode_full(case):
    dc = DeviceCase(case)
    pps = ekv().ekv_decode_plan_pages_per_split(case.seq_lens, case.num_kv_heads)
    out, lse = dc.decode(torch.float32, pages_per_split=pps)
    want, wlse = oracle_decode(case)
    assert_close(out, want)
    assert_lse_close(lse, wlse)
    return out


def test_compact_decode_b32_ctx8192():
    step("fullsize compact decode B=32 ctx 8192")
    _decode_full(synth.compact_decode_case(seed=2))


def test_mixed_decode_b64_ragged_with_outliers():
    step("fullsize mixed decode B=64 ctx U[1024,16384], 30% compact, 1% x20 outliers")
    c = synth.mixed_decode_case(seed=3)
    _decode_full(c)


def _sample_rows(L, rng, extra=6):
    rows = [r for r in SAMPLE_ROWS if r < L]
    rows += list(rng.choice(L, size=min(extra, L), replace=False))
    return sorted(set(int(r) for r in rows))


def test_compact_prefill_32x8192_in_four_chunks():
    step("fullsize compact prefill 32 x 8192, 4 chunks of 4096 pages")
    pc = synth.compact_prefill_case(seed=4)
    c = pc.paged
    dc = DeviceCase(c)
    H, D, Hq = c.num_kv_heads, c.head_dim, c.num_q_heads
    ws_k = torch.empty((4096, 16, H, D), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    rng = np.random.default_rng(44)
    for chunk in range(4):
        prompts = list(range(8 * chunk, 8 * chunk + 8))
        ids, kv_start = pc.chunk_pages(prompts)
        assert ids.size == 4096
        step(f"chunk {chunk}: gather 4096 pages")
        ekv().ekv_gather_compact_pages(dc.kv(), dev(ids), True, ws_k, ws_v)
        rows = np.arange(pc.cu_seqlens_q[prompts[0]], pc.cu_seqlens_q[prompts[-1] + 1])
        q = dev(c.q[rows])
        cu = (pc.cu_seqlens_q[prompts[0]:prompts[-1] + 2] - pc.cu_seqlens_q[prompts[0]]).astype(np.int32)
        out = torch.empty((rows.size, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((rows.size, Hq), dtype=torch.float32, device="cuda")
        step(f"chunk {chunk}: prefill 8 x 8192")
        ekv().ekv_prefill_attention(q, ws_k, ws_v, dev(cu), dev(kv_start), 8192, c.sm_scale, out, lse)
        torch.cuda.synchronize()
        if chunk == 0:  # the kernel is deterministic: repeated launches give the same bits
            again = torch.empty_like(out)
            for _ in range(3):
                ekv().ekv_prefill_attention(q, ws_k, ws_v, dev(cu), dev(kv_start), 8192, c.sm_scale, again)
                torch.cuda.synchronize()
                assert torch.equal(again.view(torch.int32), out.view(torch.int32))
        wk, wv = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
        if chunk == 0:  # bit-exact gather over the whole workspace
            gk, gv = ws_k.cpu().numpy(), ws_v.cpu().numpy()
            assert np.array_equal(gk.view(np.uint16), wk.view(np.uint16))
            assert np.array_equal(gv.view(np.uint16), wv.view(np.uint16))
        sample = []
        for i, pidx in enumerate(prompts):
            sample += [int(cu[i]) + r for r in _sample_rows(8192, rng)]
        sample = np.array(sample)
        got = out[dev(sample).long()].cpu().numpy()
        glse = lse[dev(sample).long()].cpu().numpy()
        want, wlse = oracle.prefill_attention(c.q[rows], wk.reshape(-1, H, D), wv.reshape(-1, H, D),
                                              cu, kv_start, True, c.sm_scale, rows=sample)
        assert_close(got, want[sample], what=f"chunk {chunk} prefill rows")
        assert_lse_close(glse, wlse[sample])
        del out, lse, q


N_LAYERS = 36


def _route(kv, a, ws_k, ws_v, out, lse, scratch, sm_scale, side=None):
    """One mixed-batch layer on the device: gather the fresh prompts' pages into the shared
    workspace, causal prefill into rows n_decode.., decode into rows 0..n_decode-1 -- on one
    stream, or with the decode on ``side`` beside the gather + prefill."""
    nd = a["q_decode"].shape[0]
    main = torch.cuda.current_stream()
    dec_stream = main if side is None else side
    if side is not None:
        side.wait_stream(main)  # inputs and output buffers are ready
    ekv().ekv_gather_compact_pages(kv, a["ids"], True, ws_k, ws_v, stream=main)
    ekv().ekv_prefill_attention(a["q_prefill"], ws_k, ws_v, a["cu_seqlens_q"], a["kv_start"], a["prompt_len"],
                                sm_scale, out[nd:], lse[nd:], stream=main)
    ekv().ekv_decode_attention(kv, a["q_decode"], a["page_table"], a["fidelity"], a["seq_lens"], a["max_len"],
                               sm_scale, out[:nd], lse[:nd], scratch, pages_per_split=a["pps"],
                               stream=dec_stream)
    if side is not None:
        main.wait_stream(side)


def test_mixed_batch_36_layers_one_workspace():
    """Every layer of the 36-layer mixed batch (seed 5000 + layer) routed as a serving step
    routes it, through ONE workspace, one decode scratch and one output tensor reused layer
    after layer: per layer, the gathered workspace is bit-exact, every decode row and sampled
    prefill rows match the oracle, and every row is written by its own path.  Layer 0 is
    also routed with its decode on a second stream beside the gather + prefill (same bits).

    Host input generation and the oracle (about a minute of CPU per layer) run in worker
    processes a few layers ahead; the GPU side uploads, launches and compares."""
    import concurrent.futures
    import multiprocessing
    import shutil

    import mixed_layers

    H, D, Hq, nd, T = 8, 128, 32, 32, 4 * 2048
    ws_k = torch.empty((4096, 16, H, D), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    out = torch.empty((nd + T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((nd + T, Hq), dtype=torch.float32, device="cuda")
    scratch_bytes = max(ekv().ekv_decode_scratch_bytes(nd, Hq, H, D, 32768, ekv().DECODE_BALANCED),
                        ekv().ekv_decode_scratch_bytes(nd, Hq, H, D, 32768, 0))
    scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device="cuda")
    workers = max(1, min(14, (os.cpu_count() or 2) - 2))
    ahead = workers + 2
    spool = mixed_layers.spool_dir(ahead)
    ex = concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=multiprocessing.get_context("spawn"))
    worst = [0.0, 0.0]
    try:
        pending = {li: ex.submit(mixed_layers.prepare_layer, li, spool, 5 + li)
                   for li in range(min(N_LAYERS, ahead))}
        for li in range(N_LAYERS):
            path, layout, e = pending.pop(li).result()
            if li + ahead < N_LAYERS:
                pending[li + ahead] = ex.submit(mixed_layers.prepare_layer, li + ahead, spool, 5 + li + ahead)
            step(f"mixed batch layer {li}: upload, gather -> prefill -> decode through the shared workspace")
            h = mixed_layers.load_layer(path, layout)
            a = {k: dev(h[k]) for k in ("k_target", "v_target", "k_compact", "v_compact", "v_scale", "page_table",
                                        "fidelity", "seq_lens", "q_decode", "q_prefill", "cu_seqlens_q", "ids",
                                        "kv_start")}
            ws_want_k, ws_want_v = dev(h["ws_k"]), dev(h["ws_v"])
            lens = np.array(h["seq_lens"])
            del h
            os.unlink(path)
            a.update(max_len=e["max_len"], prompt_len=e["prompt_len"],
                     pps=ekv().ekv_decode_plan_pages_per_split(lens, H))
            assert ekv().ekv_decode_scratch_bytes(nd, Hq, H, D, e["max_len"], a["pps"]) <= scratch_bytes
            kv = ekv().paged_kv(H, D, a["k_target"], a["v_target"], a["k_compact"], a["v_compact"], a["v_scale"])
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            _route(kv, a, ws_k, ws_v, out, lse, scratch, e["sm_scale"])
            torch.cuda.synchronize()
            n = a["ids"].shape[0]
            assert torch.equal(ws_k[:n].view(torch.int16), ws_want_k.view(torch.int16)), f"layer {li}: workspace K"
            assert torch.equal(ws_v[:n].view(torch.int16), ws_want_v.view(torch.int16)), f"layer {li}: workspace V"
            o, ls = out.cpu().numpy(), lse.cpu().numpy()
            assert np.all(np.isfinite(o)) and np.all(np.isfinite(ls)), f"layer {li}: every row written by its path"
            d_err = assert_close(o[:nd], e["dec"], what=f"layer {li} decode rows")
            assert_lse_close(ls[:nd], e["dec_lse"])
            p_err = assert_close(o[nd:][e["sample"]], e["pre"], what=f"layer {li} prefill rows")
            assert_lse_close(ls[nd:][e["sample"]], e["pre_lse"])
            worst = [max(worst[0], d_err), max(worst[1], p_err)]
            print(f"layer {li}: decode max-abs {d_err:.2e}, prefill max-abs {p_err:.2e}", flush=True)
            if li == 0:
                step("mixed batch layer 0: decode on a second stream")
                out2, lse2 = torch.full_like(out, float("nan")), torch.full_like(lse, float("nan"))
                _route(kv, a, ws_k, ws_v, out2, lse2, scratch, e["sm_scale"], side=torch.cuda.Stream())
                torch.cuda.synchronize()
                assert torch.equal(out2.view(torch.int32), out.view(torch.int32))
                assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32))
                del out2, lse2
            del a, kv, ws_want_k, ws_want_v
    finally:
        ex.shutdown(wait=False, cancel_futures=True)
        shutil.rmtree(spool, ignore_errors=True)
    print(f"all {N_LAYERS} layers: worst decode max-abs {worst[0]:.2e}, prefill {worst[1]:.2e}", flush=True)


def test_writer_quantizes_32x8192_prompts_into_16384_pages():
    """The prefill writer at full size, in the bench's launch: sampled pages bit-exact against
    the oracle; on every page, K equals the source rows and each head's peak code is +-448."""
    step("fullsize writer: quantize 32 x 8192 prompt rows into 16,384 compact pages")
    c = synth.writer_prefill_case(seed=4)
    H, D = c.num_kv_heads, c.head_dim
    kr, vr = dev(c.k_rows), dev(c.v_rows)
    kc = torch.empty((c.n_compact_pages, 16, H, D), dtype=torch.float16, device="cuda")
    vc = torch.empty((c.n_compact_pages, 16, H, D), dtype=torch.uint8, device="cuda")
    sc = torch.empty((c.n_compact_pages, H), dtype=torch.float32, device="cuda")
    kv = ekv().paged_kv(H, D, k_compact=kc, v_compact=vc, v_scale=sc)
    dst = dev(c.dst_pages)
    ekv().ekv_quantize_pages(kv, kr, vr, dev(c.row_start), dst, dev(c.n_valid))
    torch.cuda.synchronize()
    idx = dst.long()
    assert torch.equal(kc[idx].view(torch.int16).reshape(-1), kr.view(torch.int16).reshape(-1))
    peak = (vc[idx] & 0x7F).amax(dim=(1, 3))
    assert bool((peak == 0x7E).all())
    rng = np.random.default_rng(46)
    sample = np.concatenate([[0, 1, len(c.dst_pages) - 1], rng.choice(len(c.dst_pages), 61, replace=False)])
    got_k = kc[idx[dev(sample).long()]].cpu().numpy()
    got_v = vc[idx[dev(sample).long()]].cpu().numpy()
    got_s = sc[idx[dev(sample).long()]].cpu().numpy()
    K, V, S = oracle.quantize_pages(c.k_rows, c.v_rows, c.row_start[sample], c.n_valid[sample])
    assert np.array_equal(got_k.view(np.uint16), K.view(np.uint16))
    assert np.array_equal(got_v, V)
    assert np.array_equal(got_s.view(np.uint32), S.view(np.uint32))


def test_paged_prefill_32x8192_one_launch():
    """Direct paged prefill of all 32 prompts in one launch (the bench's call): sampled rows
    against the oracle, and the first 8 prompts bit-equal to the gather route's chunk."""
    step("fullsize paged prefill 32 x 8192, one launch")
    pc = synth.compact_prefill_case(seed=4)
    c = pc.paged
    dc = DeviceCase(c)
    H, D, Hq = c.num_kv_heads, c.head_dim, c.num_q_heads
    T = int(pc.cu_seqlens_q[-1])
    out = torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_paged_attention(dc.kv(), dc.q, dev(pc.cu_seqlens_q), dc.page_table, None, 8192,
                                      c.sm_scale, out, lse)
    torch.cuda.synchronize()
    step("gather route, chunk 0, for bit comparison")
    prompts = list(range(8))
    ids, kv_start = pc.chunk_pages(prompts)
    ws_k = torch.empty((4096, 16, H, D), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    ekv().ekv_gather_compact_pages(dc.kv(), dev(ids), True, ws_k, ws_v)
    r1 = int(pc.cu_seqlens_q[8])
    g_out = torch.empty((r1, Hq, D), dtype=torch.float32, device="cuda")
    g_lse = torch.empty((r1, Hq), dtype=torch.float32, device="cuda")
    ekv().ekv_prefill_attention(dc.q[:r1], ws_k, ws_v, dev(pc.cu_seqlens_q[:9]), dev(kv_start), 8192,
                                c.sm_scale, g_out, g_lse)
    torch.cuda.synchronize()
    assert torch.equal(out[:r1].view(torch.int32), g_out.view(torch.int32))
    assert torch.equal(lse[:r1].view(torch.int32), g_lse.view(torch.int32))
    del g_out, g_lse, ws_k, ws_v
    rng = np.random.default_rng(47)
    checked = [0, 9, 17, 31]
    local = [np.array(_sample_rows(8192, rng)) for _ in checked]
    sample = np.concatenate([int(pc.cu_seqlens_q[p]) + r for p, r in zip(checked, local)])
    got = out[dev(sample).long()].cpu().numpy()
    glse = lse[dev(sample).long()].cpu().numpy()
    # the oracle over just the checked prompts (their rows, pages and flags)
    q_sub = np.concatenate([c.q[pc.cu_seqlens_q[p]:pc.cu_seqlens_q[p + 1]] for p in checked])
    cu_sub = np.arange(len(checked) + 1, dtype=np.int32) * 8192
    rows_sub = np.concatenate([i * 8192 + r for i, r in enumerate(local)])
    want, wlse = oracle.paged_prefill_attention(q_sub, c.k_target, c.v_target, c.k_compact, c.v_compact,
                                                c.v_scale, c.page_table[checked], c.fidelity[checked],
                                                cu_sub, True, c.sm_scale, rows=rows_sub)
    assert_close(got, want[rows_sub], what="paged prefill rows")
    assert_lse_close(glse, wlse[rows_sub])


def test_elastic_decode_b32_ctx8192_structured():
    """ElasticKV layout at full size (sink pair + 512 recent tokens TARGET, the middle BASE):
    the structured path in the bench's launch, every output against the oracle."""
    step("fullsize elastic decode B=32 ctx 8192, structured TARGET-BASE-TARGET")
    e = synth.elastic_decode_case(seed=6)
    c = e.paged
    kv = ekv().paged_kv(c.num_kv_heads, c.head_dim, dev(c.k_target), dev(c.v_target))
    pps = ekv().ekv_decode_plan_pages_per_split(c.seq_lens, c.num_kv_heads)
    out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.batch, c.num_q_heads), dtype=torch.float32, device="cuda")
    ekv().ekv_decode_attention_elastic(kv, dev(c.q), dev(c.page_table), None, dev(e.base_bounds), True,
                                       dev(c.seq_lens), c.max_seq_len, c.sm_scale, out, lse,
                                       pages_per_split=pps)
    torch.cuda.synchronize()
    want, wlse = oracle_decode(c)
    assert_close(out.cpu().numpy(), want)
    assert_lse_close(lse.cpu().numpy(), wlse)

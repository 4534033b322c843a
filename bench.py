"""Benchmark: mixed-fidelity paged decode attention on one MI355X.

Headline workload: compact decode, batch 32, context 8192, 32 query / 8 KV
heads, head dim 128, 16-token pages, FP16 K + E4M3 V with per-page-head fp32
scales, seeded synthetic N(0,1) data, page table a random permutation of a
17,408-page pool.  One step = one ekv_decode_attention call over the whole
batch (one split per sequence and KV head: the split kernel writes the
output), with the per-page fidelity flags read.

Prints ONE JSON line: decode HBM GB/s (algorithmic bytes / step time), with
tokens/s, a roofline object for the decode call and the CPU oracle timed on
the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode attention HBM GB/s (% of peak) + tokens/s, B=32 ctx 8K K16/V8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # a few hundred untimed calls let the part reach its sustained clocks (measured:
    # 5 warmup calls read 2% slow against 50-2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies", type=int, default=2,
                    help="pool copies rotated across steps so no step re-reads cached pages")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--no-flags", action="store_true", help="single-pool path (no per-page flag reads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle wall time")
    ap.add_argument("--workload", choices=("decode", "prefill", "mixed", "writer", "elastic"),
                    default="decode",
                    help="decode: the headline line; prefill: 32 x 8192 compact-prefill route "
                         "(gather + causal prefill, 4 chunks); mixed: the 36-layer mixed batch; "
                         "writer: cache writer (page quantizer over the 32 x 8192 prompt rows, "
                         "TARGET append); elastic: ElasticKV BASE decode (structured and general "
                         "paths) and the demotion pack")
    ap.add_argument("--layers", type=int, default=36, help="mixed workload: layers per step")
    ap.add_argument("--streams", choices=("1", "both"), default="both",
                    help="mixed workload: time the one-stream routing only, or also the two-stream one")
    ap.add_argument("--distinct-layers", type=int, default=4,
                    help="mixed workload: distinct generated layers cycled over the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for 1 GiB in, 1 GiB out."""
    import torch

    src = torch.ones(1 << 29, dtype=torch.float16, device="cuda")  # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every workload runs on a single MI355X.  Sequences and "
              "KV heads would shard across GPUs with no exchange inside attention; that is not "
              "implemented.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload == "prefill":
        bench_prefill(args)
        return
    if args.workload == "mixed":
        bench_mixed(args)
        return
    if args.workload == "writer":
        bench_writer(args)
        return
    if args.workload == "elastic":
        bench_elastic(args)
        return

    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    t0 = time.time()
    case = synth.compact_decode_case(seed=2)
    gen_s = time.time() - t0
    B, Hq, Hkv, D = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    copies = []
    for _ in range(max(1, args.copies)):
        copies.append(dict(k=dev(case.k_compact), v=dev(case.v_compact), s=dev(case.v_scale)))
    q = dev(case.q)
    pt = dev(case.page_table)
    fl = None if args.no_flags else dev(case.fidelity)
    lens = dev(case.seq_lens)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    # split plan from the host-side lengths the scheduler holds
    pps = args.pages_per_split or ekv.ekv_decode_plan_pages_per_split(case.seq_lens, Hkv)
    scratch_bytes = ekv.ekv_decode_scratch_bytes(B, Hq, Hkv, D, case.max_seq_len, pps)
    scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device="cuda")
    kvs = [ekv.paged_kv(Hkv, D, k_compact=c["k"], v_compact=c["v"], v_scale=c["s"]) for c in copies]
    stream = torch.cuda.current_stream()

    def step(i):
        ekv.ekv_decode_attention(kvs[i % len(kvs)], q, pt, fl, lens, case.max_seq_len, case.sm_scale,
                                 out, None, scratch, pages_per_split=pps, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps between two events on the launch stream;
    # the average launch duration is the region's event time / K (events between
    # the calls would add their own dispatch gaps to every call)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    region_ms = ev0.elapsed_time(ev1)

    algo_bytes = bytemodel.decode_bytes(case.seq_lens, case.fidelity, Hq, Hkv, D, out_bytes=2,
                                        lse=False, flags_read=fl is not None)
    ms_per_step = wall * 1e3 / args.steps
    value = algo_bytes / (ms_per_step * 1e-3) / 1e9
    kernel_ms = region_ms / args.steps
    achieved = algo_bytes / (kernel_ms * 1e-3) / 1e9
    single_split = -(-int(case.max_seq_len) // 16) <= pps

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, algo_bytes, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "compact paged decode: batch 32, context 8192, 32 q / 8 KV heads, head dim 128, "
                        "page 16, FP16 K + E4M3 V + fp32 page-head scales, 17,408-page pool (seed 2)",
            "batch": B, "context": int(case.seq_lens[0]), "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "page_size": 16, "fidelity_flags_read": fl is not None,
            "pages_per_split": pps,
            "pool_copies_rotated": len(kvs), "out_dtype": "f16",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": int(algo_bytes),
        "roofline": {
            "bound": "hbm",
            "kernel": ("ekv_decode_attention (decode_splitk_kernel, one split per sequence)" if single_split
                       else "ekv_decode_attention (decode_splitk_kernel + decode_merge_kernel)"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": counted_traffic(pps) if fl is not None else None,
            "avg_call_us": round(kernel_ms * 1e3, 2),
        },
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


MFMA_FP16_PEAK_TFLOPS = 2500.0


def _events(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def measured_gemm_tflops(reps=20):
    """A second denominator for the prefill: the best fp16 GEMM rate torch (hipBLASLt) reaches
    on this part, fp32 accumulation, contiguous operands, median over reps of each of three
    large shapes (m = n, k); returns (TFLOP/s, "m x n x k")."""
    import torch

    best = (0.0, "")
    for n, k in ((8192, 8192), (8192, 16384), (16384, 16384)):
        a = torch.randn((n, k), device="cuda").half()
        b = torch.randn((k, n), device="cuda").half()
        c = torch.empty((n, n), dtype=torch.float16, device="cuda")
        for _ in range(5):
            torch.mm(a, b, out=c)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            (e0, e1), = _events(1)
            e0.record()
            torch.mm(a, b, out=c)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        del a, b, c
        tf = 2.0 * n * n * k / (float(np.median(ms)) * 1e-3) / 1e12
        if tf > best[0]:
            best = (tf, f"{n} x {n} x {k}")
    return best


def bench_prefill(args):
    """Compact-prefill route, 32 fresh prompts x 8192 tokens: per 4,096-page chunk of 8
    prompts, gather (K copy + E4M3 -> FP16 with scales) then causal FP16 prefill."""
    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    pc = synth.compact_prefill_case(seed=4)
    c = pc.paged
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    H, D, Hq = c.num_kv_heads, c.head_dim, c.num_q_heads
    kv = ekv.paged_kv(H, D, k_compact=dev(c.k_compact), v_compact=dev(c.v_compact), v_scale=dev(c.v_scale))
    q = dev(c.q)
    out = torch.empty((q.shape[0], Hq, D), dtype=torch.float16, device="cuda")
    ws_k = torch.empty((4096, 16, H, D), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    chunks = []
    for ch in range(4):
        prompts = list(range(8 * ch, 8 * ch + 8))
        ids, kv_start = pc.chunk_pages(prompts)
        r0, r1 = int(pc.cu_seqlens_q[prompts[0]]), int(pc.cu_seqlens_q[prompts[-1] + 1])
        cu = (pc.cu_seqlens_q[prompts[0]:prompts[-1] + 2] - r0).astype(np.int32)
        chunks.append((dev(ids), dev(kv_start), dev(cu), r0, r1))
    stream = torch.cuda.current_stream()

    def run(evg=None, evp=None):
        for i, (ids, ks, cu, r0, r1) in enumerate(chunks):
            if evg: evg[i][0].record(stream)
            ekv.ekv_gather_compact_pages(kv, ids, True, ws_k, ws_v, stream=stream)
            if evg: evg[i][1].record(stream)
            if evp: evp[i][0].record(stream)
            ekv.ekv_prefill_attention(q[r0:r1], ws_k, ws_v, cu, ks, 8192, c.sm_scale, out[r0:r1],
                                      stream=stream)
            if evp: evp[i][1].record(stream)

    for _ in range(max(1, min(args.warmup, 20) // 2)):
        run()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 10))
    g_ms, p_ms = [], []
    t0 = time.perf_counter()
    for _ in range(steps):
        evg, evp = _events(4), _events(4)
        run(evg, evp)
        torch.cuda.synchronize()
        g_ms += [a.elapsed_time(b) for a, b in evg]
        p_ms += [a.elapsed_time(b) for a, b in evp]
    wall = (time.perf_counter() - t0) / steps
    # direct route: all 32 prompts from their pages in one launch, no workspace
    pt, cu_all = dev(c.page_table), dev(pc.cu_seqlens_q)

    def run_paged():
        ekv.ekv_prefill_paged_attention(kv, q, cu_all, pt, None, 8192, c.sm_scale, out, stream=stream)

    for _ in range(max(1, min(args.warmup, 20) // 2)):
        run_paged()
    torch.cuda.synchronize()
    d_ms = []
    for _ in range(steps):
        (a, b), = _events(1)
        a.record(stream)
        run_paged()
        b.record(stream)
        torch.cuda.synchronize()
        d_ms.append(a.elapsed_time(b))
    d = float(np.mean(d_ms)) * 1e-3
    gemm, gemm_shape = measured_gemm_tflops()
    rd, wr = bytemodel.gather_bytes(4096, H, D)
    flops = bytemodel.prefill_flops([8192] * 8, Hq, D, causal=True)
    g = float(np.mean(g_ms)) * 1e-3
    p = float(np.mean(p_ms)) * 1e-3
    line = {
        "metric": "compact-prefill route: gather HBM GB/s + causal prefill TFLOP/s",
        "value": round(flops / p / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "ms_per_step": round(wall * 1e3, 3), "higher_is_better": True, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "compact prefill: 32 fresh prompts x 8192 tokens, 32 q / 8 KV heads, "
                               "head dim 128, causal, 4,096-page workspace, 4 chunks of 8 prompts (seed 4)"},
        "prefill": {"avg_chunk_ms": round(p * 1e3, 3), "flops_per_chunk": flops,
                    "tflops": round(flops / p / 1e12, 1), "peak_tflops": MFMA_FP16_PEAK_TFLOPS,
                    "mfma_frac": round(flops / p / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                    "measured_gemm_tflops": round(gemm, 1),
                    "frac_of_measured_gemm": round(flops / p / 1e12 / gemm, 4),
                    "gemm": f"torch.mm fp16 {gemm_shape} (hipBLASLt), best of three large shapes, "
                            "same process, median of 20 each"},
        "gather": {"avg_chunk_us": round(g * 1e6, 1), "bytes_per_chunk": rd + wr,
                   "gbps": round((rd + wr) / g / 1e9, 1), "peak_gbps": HBM_PEAK_GBPS,
                   "frac": round((rd + wr) / g / 1e9 / HBM_PEAK_GBPS, 4)},
        "direct_paged": {"kernel": "ekv_prefill_paged_attention (prefill_ws128_kernel, paged source)",
                         "prompts_per_launch": 32, "avg_ms": round(d * 1e3, 3),
                         "tflops": round(4 * flops / d / 1e12, 1),
                         "mfma_frac": round(4 * flops / d / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                         "gather_route_ms_same_work": round(4 * (g + p) * 1e3, 3),
                         "speedup_vs_gather_route": round(4 * (g + p) / d, 4)},
    }
    print(json.dumps(line), flush=True)


def bench_mixed(args):
    """Mixed batch: per layer, gather the 4 fresh prompts' pages, causal prefill (rows 32..),
    then mixed-fidelity decode of the 32 running sequences (rows 0..31), one stream."""
    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    layers = []
    for li in range(max(1, args.distinct_layers)):
        L = synth.mixed_batch_layer(li)
        c = L.paged
        H, D, Hq, nd = c.num_kv_heads, c.head_dim, c.num_q_heads, L.n_decode
        prompts = range(nd, nd + len(L.prompt_lens))
        ids = np.concatenate([c.page_table[p, :(int(c.seq_lens[p]) + 15) // 16] for p in prompts]).astype(np.int32)
        ks = np.concatenate([[0], np.cumsum((L.prompt_lens + 15) // 16 * 16)[:-1]]).astype(np.int32)
        lens = c.seq_lens[:nd]
        layers.append(dict(
            kv=ekv.paged_kv(H, D, dev(c.k_target), dev(c.v_target), dev(c.k_compact), dev(c.v_compact),
                            dev(c.v_scale)),
            q=dev(np.concatenate([L.q_decode, L.q_prefill])), ids=dev(ids), ks=dev(ks),
            cu=dev(L.cu_seqlens_q), pt=dev(c.page_table[:nd]), fl=dev(c.fidelity[:nd]), lens=dev(lens),
            max_len=int(lens.max()), pps=ekv.ekv_decode_plan_pages_per_split(lens, H),
            dec_bytes=bytemodel.decode_bytes(lens, c.fidelity[:nd], Hq, H, D, out_bytes=2),
            flops=bytemodel.prefill_flops(L.prompt_lens, Hq, D), sm=c.sm_scale,
            plen=int(L.prompt_lens.max())))
        del L, c
    H, D, Hq, nd = 8, 128, 32, 32
    T = layers[0]["q"].shape[0]
    out = torch.empty((T, Hq, D), dtype=torch.float16, device="cuda")
    ws_k = torch.empty((4096, 16, H, D), dtype=torch.float16, device="cuda")
    ws_v = torch.empty_like(ws_k)
    scratch = torch.empty(max(ekv.ekv_decode_scratch_bytes(nd, Hq, H, D, l["max_len"], l["pps"])
                              for l in layers), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # Two-stream variant: the decode of each layer runs on a second stream
    # (default priority) beside that layer's gather + prefill, and the layer
    # ends when both have (the next layer's inputs depend on this layer's
    # output).  The two paths write disjoint output rows and share nothing.
    side = torch.cuda.Stream()
    fork = [torch.cuda.Event() for _ in range(args.layers)]
    join = [torch.cuda.Event() for _ in range(args.layers)]

    def step(two_streams=False):
        for li in range(args.layers):
            l = layers[li % len(layers)]
            dec_stream = stream
            if two_streams:
                fork[li].record(stream)
                side.wait_event(fork[li])
                dec_stream = side
            ekv.ekv_gather_compact_pages(l["kv"], l["ids"], True, ws_k, ws_v, stream=stream)
            ekv.ekv_prefill_attention(l["q"][nd:], ws_k, ws_v, l["cu"], l["ks"], l["plen"], l["sm"],
                                      out[nd:], stream=stream)
            ekv.ekv_decode_attention(l["kv"], l["q"][:nd], l["pt"], l["fl"], l["lens"], l["max_len"],
                                     l["sm"], out[:nd], None, scratch, pages_per_split=l["pps"],
                                     stream=dec_stream)
            if two_streams:
                join[li].record(side)
                stream.wait_event(join[li])

    steps = max(1, min(args.steps, 20))

    def timed(two_streams):
        for _ in range(max(1, min(args.warmup, 20))):
            step(two_streams)
        torch.cuda.synchronize()
        e0, e1 = _events(1)[0]
        e0.record(stream)
        for _ in range(steps):
            step(two_streams)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(False)
    ms2 = timed(True) if args.streams == "both" else None
    dec_bytes = sum(layers[li % len(layers)]["dec_bytes"] for li in range(args.layers))
    line = {
        "metric": "mixed batch step time (36 layers: gather + prefill + mixed-fidelity decode)",
        "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": steps, "higher_is_better": False,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"mixed batch: {args.layers} layers ({len(layers)} distinct seeded layers "
                               "cycled), 32 decoding requests ctx U[4096,32768] 30% compact pages + 4 fresh "
                               "prompts x 2048 on the gather+prefill route, 32 q / 8 KV heads, head dim 128"},
        "tokens_per_s": {"decode": round(nd / (ms * 1e-3), 1),
                         "prefill": round(4 * 2048 / (ms * 1e-3), 1)},
        "decode_bytes_per_step": int(dec_bytes),
    }
    if ms2 is not None:
        line["two_streams"] = {"ms": round(ms2, 3), "speedup": round(ms / ms2, 4),
                               "what": "each layer's decode on a second stream beside its gather + prefill, "
                                       "joined before the next layer"}
    print(json.dumps(line), flush=True)


def bench_writer(args):
    """Cache writer: quantize the 32 x 8192 prompt rows (FP16 K/V) into 16,384 compact pages
    (K16 + E4M3 V + page-head scales), and append rows into TARGET pages (a 32-token decode
    step, and one 65,536-token chunk of prompt rows)."""
    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    t0 = time.time()
    c = synth.writer_prefill_case(seed=4)
    gen_s = time.time() - t0
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    H, D = c.num_kv_heads, c.head_dim
    kr, vr = dev(c.k_rows), dev(c.v_rows)
    kc = torch.empty((c.n_compact_pages, 16, H, D), dtype=torch.float16, device="cuda")
    vc = torch.empty((c.n_compact_pages, 16, H, D), dtype=torch.uint8, device="cuda")
    sc = torch.empty((c.n_compact_pages, H), dtype=torch.float32, device="cuda")
    rs, dst, nv = dev(c.row_start), dev(c.dst_pages), dev(c.n_valid)
    n_pages = int(c.row_start.size)
    # TARGET pool for the appends: 4,096 pages, slots a seeded permutation
    n_t = 4096
    kt = torch.empty((n_t, 16, H, D), dtype=torch.float16, device="cuda")
    vt = torch.empty_like(kt)
    kv = ekv.paged_kv(H, D, kt, vt, kc, vc, sc)
    slots = np.random.default_rng(40).permutation(n_t * 16).astype(np.int32)
    chunk_tok = 65536
    slot_chunk, slot_step = dev(slots[:chunk_tok]), dev(slots[:32])
    assert slot_step.numel() == 32
    k_step, v_step = kr[:32].contiguous(), vr[:32].contiguous()
    stream = torch.cuda.current_stream()

    def timed(fn, steps):  # seconds per call: back-to-back calls between two events
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        (a, b), = _events(1)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / steps

    steps = max(1, min(args.steps, 20))
    tq = timed(lambda: ekv.ekv_quantize_pages(kv, kr, vr, rs, dst, nv, stream=stream), steps)
    ta = timed(lambda: ekv.ekv_append_tokens(kv, kr[:chunk_tok], vr[:chunk_tok], slot_chunk,
                                             stream=stream), steps)
    td = timed(lambda: ekv.ekv_append_tokens(kv, k_step, v_step, slot_step, stream=stream), steps)
    qr, qw = bytemodel.quantize_bytes(c.n_valid, H, D)
    ar, aw = bytemodel.append_bytes(chunk_tok, H, D)
    gbps = (qr + qw) / tq / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # CPU baseline leg only

        reps, sample = 0, 64
        t1 = time.perf_counter()
        while True:
            oracle.quantize_pages(c.k_rows, c.v_rows, c.row_start[:sample], c.n_valid[:sample])
            reps += 1
            el = time.perf_counter() - t1
            if el >= args.cpu_seconds / 2:
                break
        sr, sw = bytemodel.quantize_bytes(c.n_valid[:sample], H, D)
        cpu = {"value": round((sr + sw) * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the first {sample} of the 16,384 pages quantized {reps}x by the oracle "
                         f"in {el:.1f} s (numpy, one thread)"}
    line = {
        "metric": "cache writer: page-quantizer HBM GB/s (FP16 rows -> K16 + E4M3 V pages)",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(tq * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16->e4m3", "data": "synthetic",
        "config": {"workload": "cache writer: 32 prompts x 8192 tokens of FP16 K/V rows (8 KV heads, "
                               "head dim 128, seed 4) quantized into 16,384 compact pages of a "
                               "17,408-page pool; TARGET append of 65,536 rows and of a 32-token "
                               "decode step into a 4,096-page pool",
                   "pages": n_pages, "num_kv_heads": H, "head_dim": D},
        "roofline": {"bound": "hbm", "kernel": "ekv_quantize_pages (quantize_kernel<128>)",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_call_us": round(tq * 1e6, 2), "algorithmic_bytes": qr + qw},
        "append": {"tokens": chunk_tok, "avg_call_us": round(ta * 1e6, 2),
                   "gbps": round((ar + aw) / ta / 1e9, 1),
                   "frac": round((ar + aw) / ta / 1e9 / HBM_PEAK_GBPS, 4),
                   "decode_step_32_tokens_us": round(td * 1e6, 2)},
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


def bench_elastic(args):
    """ElasticKV BASE decode, B 32 x context 8192 (sink pair and 512 recent tokens TARGET,
    the middle 478 pages BASE): the structured path (per-sequence bounds), the general path
    (per-page flags), all-TARGET decode of the same batch for reference, and the pack."""
    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    t0 = time.time()
    e = synth.elastic_decode_case(seed=6)
    gen_s = time.time() - t0
    c = e.paged
    B, Hq, Hkv, D = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = ekv.paged_kv(Hkv, D, dev(c.k_target), dev(c.v_target))
    q, pt, fl, lens, bounds = dev(c.q), dev(c.page_table), dev(c.fidelity), dev(c.seq_lens), dev(e.base_bounds)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    pps = ekv.ekv_decode_plan_pages_per_split(c.seq_lens, Hkv)
    scratch = torch.empty(ekv.ekv_decode_scratch_bytes(B, Hq, Hkv, D, c.max_seq_len, pps), dtype=torch.uint8,
                          device="cuda")
    stream = torch.cuda.current_stream()
    # the same batch with every page TARGET (fresh pools, so no cache reuse across runs)
    t = synth.make_paged_case(6, [8192] * B, Hq, Hkv, D, compact_frac=0.0)
    kv_t = ekv.paged_kv(Hkv, D, dev(t.k_target), dev(t.v_target))
    pt_t, lens_t = dev(t.page_table), dev(t.seq_lens)

    def timed(fn, steps):  # seconds per call: back-to-back calls between two events
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        (a, b), = _events(1)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / steps

    steps = max(1, min(args.steps, 50))
    for _ in range(10):  # clocks and caches up before any variant is timed
        ekv.ekv_decode_attention_elastic(kv, q, pt, fl, None, True, lens, c.max_seq_len, c.sm_scale, out, None,
                                         scratch, pps, stream)
    torch.cuda.synchronize()
    ts = timed(lambda: ekv.ekv_decode_attention_elastic(kv, q, pt, None, bounds, True, lens, c.max_seq_len,
                                                        c.sm_scale, out, None, scratch, pps, stream), steps)
    tg = timed(lambda: ekv.ekv_decode_attention_elastic(kv, q, pt, fl, None, True, lens, c.max_seq_len,
                                                        c.sm_scale, out, None, scratch, pps, stream), steps)
    tt = timed(lambda: ekv.ekv_decode_attention(kv_t, q, pt_t, None, lens_t, 8192, c.sm_scale, out, None,
                                                scratch, pps, stream), steps)
    # the all-TARGET batch forced through the general elastic path (indicator set, all flags 0)
    fl_t = dev(t.fidelity)
    tf = timed(lambda: ekv.ekv_decode_attention_elastic(kv_t, q, pt_t, fl_t, None, True, lens_t, 8192,
                                                        c.sm_scale, out, None, scratch, pps, stream), steps)
    b_s = bytemodel.decode_bytes(c.seq_lens, c.fidelity, Hq, Hkv, D, flags_read=False, bounds_read=True)
    b_g = bytemodel.decode_bytes(c.seq_lens, c.fidelity, Hq, Hkv, D, flags_read=True)
    b_t = bytemodel.decode_bytes(t.seq_lens, t.fidelity, Hq, Hkv, D, flags_read=False)
    # demotion pack of 4,096 pairs of a separate TARGET pool
    n_pairs = 4096
    torch.manual_seed(7)
    kp = torch.randn((2 * n_pairs, 16, Hkv, D), device="cuda").half()
    vp = torch.randn_like(kp)
    kv_p = ekv.paged_kv(Hkv, D, kp, vp)
    perm = torch.randperm(2 * n_pairs, device="cuda").int()
    src_a, src_b = perm[:n_pairs].contiguous(), perm[n_pairs:].contiguous()
    tp = timed(lambda: ekv.ekv_pack_base_pairs(kv_p, src_a, src_b, src_a, stream), max(1, min(steps, 10)))
    pr, pw = bytemodel.pack_bytes(n_pairs, Hkv, D)
    gb = lambda n, sec: round(n / sec / 1e9, 1)
    line = {
        "metric": "ElasticKV BASE decode HBM GB/s (structured TARGET-BASE-TARGET path), B=32 ctx 8K",
        "value": gb(b_s, ts), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ts * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "elastic decode: batch 32, context 8192, 32 q / 8 KV heads, head dim 128; "
                               "pages 0-1 and the last 32 TARGET, pages 2-479 BASE (high FP16 byte, two "
                               "pages per TARGET block) (seed 6)", "pages_per_split": pps},
        "roofline": {"bound": "hbm", "kernel": "ekv_decode_attention_elastic (structured)",
                     "achieved": gb(b_s, ts), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(b_s / ts / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_call_us": round(ts * 1e6, 2), "algorithmic_bytes": b_s},
        "tokens_per_s": round(B / ts, 1),
        "general_path": {"avg_call_us": round(tg * 1e6, 2), "gbps": gb(b_g, tg), "algorithmic_bytes": b_g},
        "all_target_same_batch": {"avg_call_us": round(tt * 1e6, 2), "gbps": gb(b_t, tt),
                                  "algorithmic_bytes": b_t, "speedup_of_structured_base": round(tt / ts, 3),
                                  "forced_general_path_us": round(tf * 1e6, 2),
                                  "bypass_speedup": round(tf / tt, 3)},
        "structured_vs_general": round(tg / ts, 3),
        "pack": {"pairs": n_pairs, "avg_call_us": round(tp * 1e6, 2), "gbps": gb(pr + pw, tp),
                 "frac": round((pr + pw) / tp / 1e9 / HBM_PEAK_GBPS, 4)},
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


def counted_traffic(pps):
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when the decode kernel code or the split plan changed since it
    was taken."""
    import re

    path = os.path.join(ROOT, "profiles", "decode_compact_b32_ctx8192_pmc.md")
    try:
        text = open(path).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        h = decode_code_hash()
    except (OSError, AttributeError, ValueError):
        return None
    same = rec.get("kernel_code_sha256") == h and rec.get("pages_per_split") == pps
    return int(rec["traffic_bytes_per_call"]) if same else None


def decode_code_hash():
    """sha256 of the decode kernel's sources with comments and whitespace removed: it
    changes when the compiled code can, not when a comment does."""
    import hashlib
    import re

    srcs = [os.path.join(ROOT, "mixed_precision_paged_amd", "csrc", f)
            for f in ("decode.hip", "ekv_device.hpp", "ekv_internal.hpp")]
    code = []
    for f in srcs:
        t = open(f).read()
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        code.append(" ".join(t.split()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def cpu_baseline(case, algo_bytes, min_seconds):
    """The float64 oracle on the host cores over the same batch, repeated to >= min_seconds."""
    import oracle  # CPU baseline leg only

    try:
        import threadpoolctl
        blas = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # threadpoolctl absent: numpy's default
        blas = os.cpu_count() or 1
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_attention(case.q, case.k_target, case.v_target, case.k_compact, case.v_compact,
                                case.v_scale, case.page_table, case.fidelity, case.seq_lens,
                                case.sm_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {
        "value": round(algo_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas),
        "host_cpu_count": os.cpu_count(),
        "kind": "oracle",
        "sample": f"the whole batch (32 sequences x 8192 tokens) decoded {reps}x by the float64 "
                  f"oracle in {el:.1f} s",
        "tokens_per_s": round(case.batch * reps / el, 3),
    }


if __name__ == "__main__":
    main()

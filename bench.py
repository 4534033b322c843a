"""Benchmark: mixed-fidelity paged decode attention on one MI355X.

Headline workload: compact decode, batch 32, context 8192, 32 query / 8 KV
heads, head dim 128, 16-token pages, FP16 K + E4M3 V with per-page-head fp32
scales, seeded synthetic N(0,1) data, page table a random permutation of a
17,408-page pool.  One step = one ekv_decode_attention call over the whole
batch (one split per sequence and KV head: the split kernel writes the
output), with the per-page fidelity flags read.

Timing of every line: an untimed clock ramp (back-to-back calls for at least
--ramp-seconds, stated in the line), the W warm-up calls, a synchronize, a few
untimed calls queued ahead of the first event (so the timed region starts on
a busy GPU, not on an idle one waiting for the host), then exactly K calls
between two events on the launch stream, and a synchronize.

Prints ONE JSON line: decode HBM GB/s (algorithmic bytes / step time), with
tokens/s, a roofline object for the decode call and the CPU oracle timed on
the host as a baseline (a process pool over (sequence, KV head) tasks, BLAS at
one thread per worker).

Other workloads (--workload): mixed-decode (batch 64 ragged mixed-fidelity
decode), prefill (32 x 8192 compact-prefill route), mixed (the 36-layer mixed
batch), writer (cache writer), elastic (ElasticKV BASE decode).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import multiprocessing
import os
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
METRIC = "decode attention HBM GB/s (% of peak) + tokens/s, B=32 ctx 8K K16/V8"
PRE_ROLL = 3           # untimed calls queued ahead of the first event
CPU_WORKERS_MAX = 16   # one GPU's share of the host cores


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--ramp-seconds", type=float, default=0.3,
                    help="untimed back-to-back calls before the warm-up, so the part runs at its "
                         "sustained clocks (5 warm-up calls alone measured 8%% slow)")
    ap.add_argument("--copies", type=int, default=2,
                    help="pool copies rotated across steps so no step re-reads cached pages")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--no-flags", action="store_true", help="single-pool path (no per-page flag reads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle wall time")
    ap.add_argument("--workload", choices=("decode", "mixed-decode", "prefill", "mixed", "writer", "elastic"),
                    default="decode",
                    help="decode: the headline line; mixed-decode: batch 64, contexts U[1024,16384], 30%% "
                         "compact pages, 1%% V outliers x20; prefill: 32 x 8192 compact-prefill route "
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


# ----------------------------------------------------------------- timing

def _events(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def clock_ramp(fn, seconds):
    """Untimed back-to-back calls for at least `seconds` of wall time; returns the call count."""
    import torch

    calls, t0 = 0, time.perf_counter()
    while True:
        for _ in range(16):
            fn(calls)
            calls += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return calls


def timed_calls(fn, steps, warmup, stream, ramp_seconds):
    """Clock ramp, `warmup` calls, a synchronize, PRE_ROLL queued calls, then exactly `steps`
    calls between two events on `stream`, and a synchronize.  fn(i) issues call i.
    Returns (seconds per call from the events, ramp calls, wall seconds of the timed block)."""
    import torch

    ramp = clock_ramp(fn, ramp_seconds) if ramp_seconds > 0 else 0
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(PRE_ROLL):
        fn(i)
    (e0, e1), = _events(1)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) * 1e-3 / steps, ramp, wall


def timing_note(ramp_calls, args):
    return {"clock_ramp_calls": ramp_calls, "clock_ramp_s": args.ramp_seconds, "pre_roll_calls": PRE_ROLL,
            "timed": "exactly `steps` calls between two HIP events on the launch stream; the ramp, "
                     "warm-up and pre-roll calls are untimed"}


# ------------------------------------------------------------ CPU baseline
# The oracle (float64 numpy, unchanged) in a spawned process pool over
# independent tasks, BLAS limited to one thread per worker.  The inputs are
# written once to a memory-mapped file that the workers map.

def _cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(CPU_WORKERS_MAX, n))


def _spool(arrays):
    base = "/dev/shm" if os.path.isdir("/dev/shm") else None
    fd, path = tempfile.mkstemp(prefix="ekv_cpu_", suffix=".bin", dir=base)
    os.close(fd)
    layout, off = {}, 0
    for name, a in arrays.items():
        a = np.ascontiguousarray(a)
        layout[name] = (off, a.dtype.str, a.shape)
        off += (a.nbytes + 255) // 256 * 256
    mm = np.memmap(path, dtype=np.uint8, mode="w+", shape=(max(off, 1),))
    for name, a in arrays.items():
        a = np.ascontiguousarray(a)
        o = layout[name][0]
        mm[o:o + a.nbytes] = a.reshape(-1).view(np.uint8)
    mm.flush()
    del mm
    return path, layout


_CPU = {}


def _cpu_init(path, layout):
    import threadpoolctl

    _CPU["_limit"] = threadpoolctl.threadpool_limits(1)
    mm = np.memmap(path, dtype=np.uint8, mode="r")
    for name, (off, dt, shape) in layout.items():
        dt = np.dtype(dt)
        n = int(np.prod(shape)) if len(shape) else 1
        _CPU[name] = mm[off:off + n * dt.itemsize].view(dt).reshape(shape)


def _pool_arg(name, heads):
    a = _CPU.get(name)
    if a is None or heads is None:
        return a
    return a[:, :, heads] if a.ndim == 4 else a[:, heads]


def _cpu_task(task):
    """One oracle task: ("decode", b, g or None, G, sm) -- sequence b, KV head g (all heads
    when None); ("prefill", p, g, G, sm, rows) -- prompt p, KV head g, query rows `rows`."""
    import oracle  # CPU baseline leg only

    c = _CPU
    if task[0] == "decode":
        _, b, g, G, sm = task
        hs = None if g is None else slice(g, g + 1)
        q = c["q"][b:b + 1] if g is None else c["q"][b:b + 1, g * G:(g + 1) * G]
        oracle.decode_attention(q, _pool_arg("k_target", hs), _pool_arg("v_target", hs),
                                _pool_arg("k_compact", hs), _pool_arg("v_compact", hs),
                                _pool_arg("v_scale", hs), c["page_table"][b:b + 1], c["fidelity"][b:b + 1],
                                c["seq_lens"][b:b + 1], sm)
    elif task[0] == "prefill":
        _, p, g, G, sm, rows = task
        cu, ks = c["cu_seqlens_q"], c["kv_start"]
        L = int(cu[p + 1] - cu[p])
        q = c["q_prefill"][int(cu[p]):int(cu[p + 1]), g * G:(g + 1) * G]
        oracle.prefill_attention(q, c["ws_k"][:, g:g + 1], c["ws_v"][:, g:g + 1], np.array([0, L]),
                                 np.array([int(ks[p])]), True, sm, rows=rows)
    elif task[0] == "quantize":
        _, lo, hi = task
        oracle.quantize_pages(c["k_rows"], c["v_rows"], c["row_start"][lo:hi], c["n_valid"][lo:hi])
    return 1


def cpu_pool_time(arrays, tasks, min_seconds):
    """Wall seconds per round of `tasks` over a spawned pool (one untimed round first),
    repeated for at least min_seconds; returns (seconds per round, rounds, workers)."""
    workers = _cpu_workers()
    path, layout = _spool(arrays)
    try:
        ctx = multiprocessing.get_context("spawn")
        with ctx.Pool(workers, initializer=_cpu_init, initargs=(path, layout)) as pool:
            pool.map(_cpu_task, tasks, chunksize=1)  # untimed: worker start-up, page mapping
            rounds, t0 = 0, time.perf_counter()
            while True:
                pool.map(_cpu_task, tasks, chunksize=1)
                rounds += 1
                el = time.perf_counter() - t0
                if el >= min_seconds:
                    break
    finally:
        os.unlink(path)
    return el / rounds, rounds, workers


def decode_arrays(case):
    return {"q": case.q, "k_target": case.k_target, "v_target": case.v_target, "k_compact": case.k_compact,
            "v_compact": case.v_compact, "v_scale": case.v_scale, "page_table": case.page_table,
            "fidelity": case.fidelity, "seq_lens": case.seq_lens}


def cpu_decode_baseline(case, algo_bytes, min_seconds, per_head=True, what="the whole batch"):
    G = case.num_q_heads // case.num_kv_heads
    heads = range(case.num_kv_heads) if per_head else [None]
    tasks = [("decode", b, g, G, case.sm_scale) for b in range(case.batch) for g in heads]
    sec, rounds, workers = cpu_pool_time(decode_arrays(case), tasks, min_seconds)
    return {"value": round(algo_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{what} ({case.batch} sequences) decoded {rounds}x by the float64 oracle in "
                      f"{sec * rounds:.1f} s, {len(tasks)} (sequence, KV head{'' if per_head else 's'}) tasks "
                      f"per round over {workers} worker processes, BLAS at one thread each",
            "tokens_per_s": round(case.batch / sec, 3), "host_cpu_count": os.cpu_count()}


# ----------------------------------------------------------------- decode

def bench_decode(args, mixed=False):
    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    t0 = time.time()
    case = synth.mixed_decode_case(seed=3) if mixed else synth.compact_decode_case(seed=2)
    gen_s = time.time() - t0
    B, Hq, Hkv, D = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    kvs = []
    for _ in range(max(1, args.copies)):
        if mixed:
            kvs.append(ekv.paged_kv(Hkv, D, dev(case.k_target), dev(case.v_target), dev(case.k_compact),
                                    dev(case.v_compact), dev(case.v_scale)))
        else:
            kvs.append(ekv.paged_kv(Hkv, D, k_compact=dev(case.k_compact), v_compact=dev(case.v_compact),
                                    v_scale=dev(case.v_scale)))
    q = dev(case.q)
    pt = dev(case.page_table)
    fl = None if (args.no_flags and not mixed) else dev(case.fidelity)
    lens = dev(case.seq_lens)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    # split plan from the host-side lengths the scheduler holds
    pps = args.pages_per_split or ekv.ekv_decode_plan_pages_per_split(case.seq_lens, Hkv)
    scratch_bytes = ekv.ekv_decode_scratch_bytes(B, Hq, Hkv, D, case.max_seq_len, pps)
    scratch = torch.empty(max(scratch_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        ekv.ekv_decode_attention(kvs[i % len(kvs)], q, pt, fl, lens, case.max_seq_len, case.sm_scale,
                                 out, None, scratch, pages_per_split=pps, stream=stream)

    sec, ramp, wall = timed_calls(step, args.steps, args.warmup, stream, args.ramp_seconds)
    algo_bytes = bytemodel.decode_bytes(case.seq_lens, case.fidelity, Hq, Hkv, D, out_bytes=2,
                                        lse=False, flags_read=fl is not None)
    gbps = algo_bytes / sec / 1e9
    n_splits = -(-(-(-int(case.max_seq_len) // 16)) // pps) if pps > 0 else 0
    if pps == ekv.DECODE_BALANCED:
        kernel = "ekv_decode_attention (decode_balanced_kernel + decode_merge_kernel)"
    elif n_splits <= 1:
        kernel = "ekv_decode_attention (decode_splitk_kernel, one split per sequence)"
    elif n_splits <= 32:
        kernel = f"ekv_decode_attention (decode_splitk_kernel, {n_splits} splits merged in the kernel)"
    else:
        kernel = "ekv_decode_attention (decode_splitk_kernel + decode_merge_kernel)"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_decode_baseline(case, algo_bytes, args.cpu_seconds)

    if mixed:
        workload = ("mixed-fidelity paged decode: batch 64, contexts U[1024,16384], 30% of pages compact "
                    "(FP16 K + E4M3 V + fp32 page-head scales) and 70% TARGET in separate pools, 1% of V "
                    "entries x20, 32 q / 8 KV heads, head dim 128, page 16 (seed 3)")
        metric = "mixed-fidelity decode attention HBM GB/s (% of peak) + tokens/s, B=64 ctx U[1K,16K]"
    else:
        workload = ("compact paged decode: batch 32, context 8192, 32 q / 8 KV heads, head dim 128, page 16, "
                    "FP16 K + E4M3 V + fp32 page-head scales, 17,408-page pool (seed 2)")
        metric = METRIC
    line = {
        "metric": metric,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "batch": B, "context": "U[1024,16384]" if mixed else int(case.seq_lens[0]), "num_q_heads": Hq,
            "num_kv_heads": Hkv, "head_dim": D, "page_size": 16, "fidelity_flags_read": fl is not None,
            "pages_per_split": pps, "pool_copies_rotated": len(kvs), "out_dtype": "f16",
        },
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B / sec, 1),
        "algorithmic_bytes_per_step": int(algo_bytes),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": None if mixed else (counted_traffic(pps) if fl is not None else None),
            "avg_call_us": round(sec * 1e6, 2),
        },
        "timing": dict(timing_note(ramp, args), wall_s_timed_block=round(wall, 4)),
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------- prefill

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


def prefill_row_flops(rows, G, D):
    """QK^T + PV FLOPs of causal query rows at positions `rows` (0-based), G query heads."""
    return int(sum(4 * D * G * (int(i) + 1) for i in rows))


def cpu_prefill_baseline(q_prefill, ws_k, ws_v, cu, kv_start, prompts, Hq, Hkv, D, sm, min_seconds,
                         rows_per_prompt=48, seed=40):
    """The oracle's causal attention on the gathered workspace rows of `prompts`, each
    (prompt, KV head) task on a uniform sample of query rows; TFLOP/s of the rows computed."""
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    tasks, flops = [], 0
    for p in prompts:
        L = int(cu[p + 1] - cu[p])
        rows = np.sort(rng.choice(L, size=min(rows_per_prompt, L), replace=False))
        for g in range(Hkv):
            tasks.append(("prefill", p, g, G, sm, rows))
            flops += prefill_row_flops(rows, G, D)
    arrays = {"q_prefill": q_prefill, "ws_k": ws_k, "ws_v": ws_v, "cu_seqlens_q": cu, "kv_start": kv_start}
    sec, rounds, workers = cpu_pool_time(arrays, tasks, min_seconds)
    return sec, flops, rounds, workers, len(tasks)


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
    steps = max(1, min(args.steps, 10))

    def run(i):  # one step = the whole prompt set: 4 x (gather, prefill)
        for ids, ks, cu, r0, r1 in chunks:
            ekv.ekv_gather_compact_pages(kv, ids, True, ws_k, ws_v, stream=stream)
            ekv.ekv_prefill_attention(q[r0:r1], ws_k, ws_v, cu, ks, 8192, c.sm_scale, out[r0:r1], stream=stream)

    sec, ramp, wall = timed_calls(run, steps, max(1, min(args.warmup, 3)), stream, args.ramp_seconds)
    # per-kernel durations: events around each gather and prefill call (separate pass)
    g_ms, p_ms = [], []
    for _ in range(steps):
        evg, evp = _events(4), _events(4)
        for i, (ids, ks, cu, r0, r1) in enumerate(chunks):
            evg[i][0].record(stream)
            ekv.ekv_gather_compact_pages(kv, ids, True, ws_k, ws_v, stream=stream)
            evg[i][1].record(stream)
            evp[i][0].record(stream)
            ekv.ekv_prefill_attention(q[r0:r1], ws_k, ws_v, cu, ks, 8192, c.sm_scale, out[r0:r1], stream=stream)
            evp[i][1].record(stream)
        torch.cuda.synchronize()
        g_ms += [a.elapsed_time(b) for a, b in evg]
        p_ms += [a.elapsed_time(b) for a, b in evp]
    # direct route: all 32 prompts from their pages in one launch, no workspace
    pt, cu_all = dev(c.page_table), dev(pc.cu_seqlens_q)

    def run_paged(i):
        ekv.ekv_prefill_paged_attention(kv, q, cu_all, pt, None, 8192, c.sm_scale, out, stream=stream)

    d, _, _ = timed_calls(run_paged, steps, 2, stream, 0.0)
    gemm, gemm_shape = measured_gemm_tflops()
    rd, wr = bytemodel.gather_bytes(4096, H, D)
    flops = bytemodel.prefill_flops([8192] * 8, Hq, D, causal=True)
    g = float(np.mean(g_ms)) * 1e-3
    p = float(np.mean(p_ms)) * 1e-3
    tflops = flops / p / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # CPU baseline leg only: the workspace values of the first 4 prompts

        ids, ks = pc.chunk_pages([0, 1, 2, 3])
        wk, wv = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
        r1 = int(pc.cu_seqlens_q[4])
        csec, cflops, rounds, workers, ntask = cpu_prefill_baseline(
            c.q[:r1], wk.reshape(-1, H, D), wv.reshape(-1, H, D), pc.cu_seqlens_q[:5], ks, range(4), Hq, H, D,
            c.sm_scale, args.cpu_seconds)
        cpu = {"value": round(cflops / csec / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
               "sample": f"48 uniformly drawn query rows of each of prompts 0-3 (8192 tokens each), every "
                         f"query head, causal attention over the gathered workspace rows, {rounds}x in "
                         f"{csec * rounds:.1f} s ({ntask} (prompt, KV head) tasks over {workers} worker "
                         f"processes, BLAS at one thread); FLOPs counted as for the GPU (QK^T + PV of the "
                         f"visible keys)",
               "host_cpu_count": os.cpu_count()}
    line = {
        "metric": "compact-prefill route: causal FP16 prefill TFLOP/s (+ gather HBM GB/s)",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": max(1, min(args.warmup, 3)),
        "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "compact prefill: 32 fresh prompts x 8192 tokens, 32 q / 8 KV heads, "
                               "head dim 128, causal, 4,096-page workspace, 4 chunks of 8 prompts (seed 4)"},
        "roofline": {"bound": "mfma", "kernel": "ekv_prefill_attention (prefill_pipe_kernel)",
                     "achieved": round(tflops, 1), "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                     "traffic": counted_prefill_traffic(),
                     "avg_call_us": round(p * 1e6, 1), "flops_per_call": flops},
        "prefill": {"avg_chunk_ms": round(p * 1e3, 3), "flops_per_chunk": flops,
                    "tflops": round(tflops, 1), "peak_tflops": MFMA_FP16_PEAK_TFLOPS,
                    "mfma_frac": round(tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                    "measured_gemm_tflops": round(gemm, 1),
                    "frac_of_measured_gemm": round(tflops / gemm, 4),
                    "gemm": f"torch.mm fp16 {gemm_shape} (hipBLASLt), best of three large shapes, "
                            "same process, median of 20 each"},
        "gather": {"avg_chunk_us": round(g * 1e6, 1), "bytes_per_chunk": rd + wr,
                   "gbps": round((rd + wr) / g / 1e9, 1), "peak_gbps": HBM_PEAK_GBPS,
                   "frac": round((rd + wr) / g / 1e9 / HBM_PEAK_GBPS, 4)},
        "direct_paged": {"kernel": "ekv_prefill_paged_attention (prefill_pipe_kernel, paged source)",
                         "prompts_per_launch": 32, "avg_ms": round(d * 1e3, 3),
                         "tflops": round(4 * flops / d / 1e12, 1),
                         "mfma_frac": round(4 * flops / d / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                         "gather_route_ms_same_work": round(sec * 1e3, 3),
                         "speedup_vs_gather_route": round(sec / d, 4)},
        "timing": dict(timing_note(ramp, args), wall_s_timed_block=round(wall, 4),
                       per_kernel="events around each gather and prefill call in a separate pass"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------- mixed batch

def bench_mixed(args):
    """Mixed batch: per layer, gather the 4 fresh prompts' pages, causal prefill (rows 32..),
    then mixed-fidelity decode of the 32 running sequences (rows 0..31), one stream."""
    import torch

    from mixed_precision_paged_amd import bytemodel, ekv, synth

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    layers = []
    first = None
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
        if li == 0 and not args.no_cpu_baseline:
            first = (L, ids, ks)
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

    def step(i, two_streams=False):
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
    warm = max(1, min(args.warmup, 5))
    sec, ramp, wall = timed_calls(step, steps, warm, stream, args.ramp_seconds)
    sec2 = None
    if args.streams == "both":
        sec2, _, _ = timed_calls(lambda i: step(i, True), steps, warm, stream, 0.0)
    # the dominant kernel: each distinct layer's decode, events around the call (separate pass)
    dec_us = []
    for l in layers:
        def dec(i, l=l):
            ekv.ekv_decode_attention(l["kv"], l["q"][:nd], l["pt"], l["fl"], l["lens"], l["max_len"], l["sm"],
                                     out[:nd], None, scratch, pages_per_split=l["pps"], stream=stream)
        dec_us.append(timed_calls(dec, 20, 3, stream, 0.0)[0])
    dec_bytes_layer = [l["dec_bytes"] for l in layers]
    dec_gbps = float(np.mean([b / s / 1e9 for b, s in zip(dec_bytes_layer, dec_us)]))
    dec_bytes = sum(layers[li % len(layers)]["dec_bytes"] for li in range(args.layers))
    pf_flops = layers[0]["flops"]

    cpu = None
    if first is not None:
        L, ids, ks = first
        c = L.paged
        G = Hq // H
        dsec, drounds, workers = cpu_pool_time(
            {"q": L.q_decode, "k_target": c.k_target, "v_target": c.v_target, "k_compact": c.k_compact,
             "v_compact": c.v_compact, "v_scale": c.v_scale, "page_table": c.page_table[:nd],
             "fidelity": c.fidelity[:nd], "seq_lens": c.seq_lens[:nd]},
            [("decode", b, g, G, c.sm_scale) for b in range(nd) for g in range(H)], args.cpu_seconds / 2)
        import oracle  # CPU baseline leg only: layer 0's gathered workspace values

        wk, wv = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
        psec, pflops_s, prounds, _, _ = cpu_prefill_baseline(
            L.q_prefill, wk.reshape(-1, H, D), wv.reshape(-1, H, D), L.cu_seqlens_q, ks,
            range(len(L.prompt_lens)), Hq, H, D, c.sm_scale, args.cpu_seconds / 2)
        layer_s = dsec + psec * pf_flops / pflops_s
        cpu = {"value": round(layer_s * args.layers * 1e3, 1), "unit": "ms", "cores": workers, "kind": "oracle",
               "sample": f"layer 0: its 32 decode rows ({drounds}x, {dsec:.2f} s each, (sequence, KV head) "
                         f"tasks) and 48 uniformly drawn query rows of each of its 4 prompts ({prounds}x, "
                         f"{psec:.3f} s each, scaled by the FLOPs of all rows), times {args.layers} layers; "
                         f"{workers} worker processes, BLAS at one thread",
               "host_cpu_count": os.cpu_count()}
    line = {
        "metric": "mixed batch step time (36 layers: gather + prefill + mixed-fidelity decode)",
        "value": round(sec * 1e3, 3), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(sec * 1e3, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"mixed batch: {args.layers} layers ({len(layers)} distinct seeded layers "
                               "cycled), 32 decoding requests ctx U[4096,32768] 30% compact pages + 4 fresh "
                               "prompts x 2048 on the gather+prefill route, 32 q / 8 KV heads, head dim 128, "
                               "one workspace, decode scratch and output tensor reused by every layer"},
        "tokens_per_s": {"decode": round(nd / sec, 1), "prefill": round(4 * 2048 / sec, 1)},
        "decode_bytes_per_step": int(dec_bytes),
        "roofline": {"bound": "hbm", "kernel": "ekv_decode_attention (balanced plan), each distinct layer",
                     "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_call_us": round(float(np.mean(dec_us)) * 1e6, 1),
                     "algorithmic_bytes_per_call": [int(b) for b in dec_bytes_layer]},
        "timing": dict(timing_note(ramp, args), wall_s_timed_block=round(wall, 4)),
        "cpu_baseline": cpu,
    }
    if sec2 is not None:
        line["two_streams"] = {"ms": round(sec2 * 1e3, 3), "speedup": round(sec / sec2, 4),
                               "what": "each layer's decode on a second stream beside its gather + prefill, "
                                       "joined before the next layer"}
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------- cache writer

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
    steps = max(1, min(args.steps, 20))
    tq, ramp, wall = timed_calls(lambda i: ekv.ekv_quantize_pages(kv, kr, vr, rs, dst, nv, stream=stream),
                                 steps, args.warmup, stream, args.ramp_seconds)
    ta, _, _ = timed_calls(lambda i: ekv.ekv_append_tokens(kv, kr[:chunk_tok], vr[:chunk_tok], slot_chunk,
                                                           stream=stream), steps, args.warmup, stream, 0.0)
    td, _, _ = timed_calls(lambda i: ekv.ekv_append_tokens(kv, k_step, v_step, slot_step, stream=stream),
                           steps, args.warmup, stream, 0.0)
    qr, qw = bytemodel.quantize_bytes(c.n_valid, H, D)
    ar, aw = bytemodel.append_bytes(chunk_tok, H, D)
    gbps = (qr + qw) / tq / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        per, n_tasks = 16, 4 * _cpu_workers()
        sample = per * n_tasks
        rows = int(c.row_start[sample - 1] + c.n_valid[sample - 1])
        csec, rounds, workers = cpu_pool_time(
            {"k_rows": c.k_rows[:rows], "v_rows": c.v_rows[:rows], "row_start": c.row_start[:sample],
             "n_valid": c.n_valid[:sample]},
            [("quantize", i * per, (i + 1) * per) for i in range(n_tasks)], args.cpu_seconds)
        sr, sw = bytemodel.quantize_bytes(c.n_valid[:sample], H, D)
        cpu = {"value": round((sr + sw) / csec / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
               "sample": f"the first {sample} of the 16,384 pages quantized by the oracle {rounds}x in "
                         f"{csec * rounds:.1f} s ({n_tasks} tasks of {per} pages over {workers} worker "
                         f"processes, BLAS at one thread)", "host_cpu_count": os.cpu_count()}
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
        "timing": dict(timing_note(ramp, args), wall_s_timed_block=round(wall, 4)),
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------- ElasticKV

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
    scratch = torch.empty(max(1, ekv.ekv_decode_scratch_bytes(B, Hq, Hkv, D, c.max_seq_len, pps)),
                          dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # the same batch with every page TARGET (fresh pools, so no cache reuse across runs)
    t = synth.make_paged_case(6, [8192] * B, Hq, Hkv, D, compact_frac=0.0)
    kv_t = ekv.paged_kv(Hkv, D, dev(t.k_target), dev(t.v_target))
    pt_t, lens_t = dev(t.page_table), dev(t.seq_lens)
    steps = max(1, min(args.steps, 50))
    ts, ramp, wall = timed_calls(
        lambda i: ekv.ekv_decode_attention_elastic(kv, q, pt, None, bounds, True, lens, c.max_seq_len, c.sm_scale,
                                                   out, None, scratch, pps, stream), steps, args.warmup, stream,
        args.ramp_seconds)
    tg, _, _ = timed_calls(
        lambda i: ekv.ekv_decode_attention_elastic(kv, q, pt, fl, None, True, lens, c.max_seq_len, c.sm_scale,
                                                   out, None, scratch, pps, stream), steps, args.warmup, stream,
        0.0)
    tt, _, _ = timed_calls(
        lambda i: ekv.ekv_decode_attention(kv_t, q, pt_t, None, lens_t, 8192, c.sm_scale, out, None, scratch, pps,
                                           stream), steps, args.warmup, stream, 0.0)
    # the all-TARGET batch forced through the general elastic path (indicator set, all flags 0)
    fl_t = dev(t.fidelity)
    tf, _, _ = timed_calls(
        lambda i: ekv.ekv_decode_attention_elastic(kv_t, q, pt_t, fl_t, None, True, lens_t, 8192, c.sm_scale,
                                                   out, None, scratch, pps, stream), steps, args.warmup, stream,
        0.0)
    b_s = bytemodel.decode_bytes(c.seq_lens, c.fidelity, Hq, Hkv, D, flags_read=False, bounds_read=True)
    b_g = bytemodel.decode_bytes(c.seq_lens, c.fidelity, Hq, Hkv, D, flags_read=True)
    b_t = bytemodel.decode_bytes(t.seq_lens, t.fidelity, Hq, Hkv, D, flags_read=False)
    del kv_t, pt_t, lens_t, fl_t, t
    # demotion pack of 4,096 pairs of a separate TARGET pool
    n_pairs = 4096
    torch.manual_seed(7)
    kp = torch.randn((2 * n_pairs, 16, Hkv, D), device="cuda").half()
    vp = torch.randn_like(kp)
    kv_p = ekv.paged_kv(Hkv, D, kp, vp)
    perm = torch.randperm(2 * n_pairs, device="cuda").int()
    src_a, src_b = perm[:n_pairs].contiguous(), perm[n_pairs:].contiguous()
    tp, _, _ = timed_calls(lambda i: ekv.ekv_pack_base_pairs(kv_p, src_a, src_b, src_a, stream),
                           max(1, min(steps, 10)), 3, stream, 0.0)
    pr, pw = bytemodel.pack_bytes(n_pairs, Hkv, D)
    gb = lambda n, sec: round(n / sec / 1e9, 1)
    cpu = None
    if not args.no_cpu_baseline:
        # BASE pages span every KV head of a block, so tasks are whole sequences
        cpu = cpu_decode_baseline(c, b_g, args.cpu_seconds, per_head=False)
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
        "timing": dict(timing_note(ramp, args), wall_s_timed_block=round(wall, 4)),
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------- counters

def pmc_record(name):
    """The JSON record of a committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None."""
    import re

    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
        return json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    except (OSError, AttributeError, ValueError):
        return None


def counted_traffic(pps):
    """HBM bytes per decode call from the committed counter summary, or None when the
    decode kernel code or the split plan changed since it was taken."""
    rec = pmc_record("decode_compact_b32_ctx8192_pmc.md")
    if rec is None:
        return None
    same = rec.get("kernel_code_sha256") == decode_code_hash() and rec.get("pages_per_split") == pps
    return int(rec["traffic_bytes_per_call"]) if same else None


def counted_prefill_traffic():
    """HBM bytes per workspace prefill call (8 x 8192 chunk) from the committed counter
    summary, or None when the prefill kernel code changed since it was taken."""
    rec = pmc_record("prefill_route_32x8192_pmc.md")
    if rec is None or rec.get("kernel_code_sha256") != prefill_code_hash():
        return None
    return int(rec["traffic_bytes_per_call"])


def decode_code_hash():
    return code_hash(("decode.hip", "ekv_device.hpp", "ekv_internal.hpp"))


def prefill_code_hash():
    return code_hash(("prefill.hip", "ekv_device.hpp", "ekv_internal.hpp"))


def code_hash(files):
    """sha256 of a kernel's sources with comments and whitespace removed: it changes
    when the compiled code can, not when a comment does."""
    import hashlib
    import re

    srcs = [os.path.join(ROOT, "mixed_precision_paged_amd", "csrc", f) for f in files]
    code = []
    for f in srcs:
        t = open(f).read()
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        code.append(" ".join(t.split()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


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
    {"decode": lambda a: bench_decode(a), "mixed-decode": lambda a: bench_decode(a, mixed=True),
     "prefill": bench_prefill, "mixed": bench_mixed, "writer": bench_writer,
     "elastic": bench_elastic}[args.workload](args)


if __name__ == "__main__":
    main()

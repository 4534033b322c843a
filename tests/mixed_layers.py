"""Host side of the 36-layer mixed-batch parity test: one layer's inputs and its
oracle expectations, prepared in a worker process (no GPU use there).

A worker generates layer ``li`` (seed 5000 + li), computes with the oracle
  * every decode row and its LSE,
  * the gathered workspace pages of the layer's fresh prompts (bit-exact contract),
  * sampled prefill rows and their LSE,
and writes the arrays the GPU needs, plus the expected workspace, into one flat
file (under /dev/shm when it has room), so the main process maps them instead of
receiving gigabytes through a pipe.  The main process deletes the file once the
arrays are on the device.
"""
from __future__ import annotations

import os
import shutil
import tempfile

import numpy as np

SAMPLE_ROWS = (0, 1, 15, 16, 63, 64, 127, 128, 129, 2047, 4095, 4096, 8190, 8191)
LAYER_BYTES = 3 << 30  # upper bound of one layer's file (inputs + expected workspace)


def sample_rows(L, rng, extra=6):
    rows = [r for r in SAMPLE_ROWS if r < L]
    rows += list(rng.choice(L, size=min(extra, L), replace=False))
    return sorted(set(int(r) for r in rows))


def spool_dir(ahead: int) -> str:
    """A directory for `ahead` layer files: /dev/shm when it has room, else the temp dir."""
    base = "/dev/shm"
    try:
        if shutil.disk_usage(base).free < (ahead + 2) * LAYER_BYTES:
            base = tempfile.gettempdir()
    except OSError:
        base = tempfile.gettempdir()
    return tempfile.mkdtemp(prefix="ekv_layers_", dir=base)


def routing_plan(L):
    """Page ids of the fresh prompts in logical order and each prompt's first workspace row."""
    c = L.paged
    nd = L.n_decode
    prompts = range(nd, nd + len(L.prompt_lens))
    ids = np.concatenate([c.page_table[p, :(int(c.seq_lens[p]) + 15) // 16] for p in prompts]).astype(np.int32)
    kv_start = np.concatenate([[0], np.cumsum((L.prompt_lens + 15) // 16 * 16)[:-1]]).astype(np.int32)
    return ids, kv_start


def prepare_layer(li: int, spool: str, seed: int):
    """Worker: returns (path, layout, expectations) for layer li.  ``layout`` maps an
    array name to (offset, dtype str, shape) inside the file at ``path``."""
    import threadpoolctl
    import torch

    torch.set_num_threads(1)
    with threadpoolctl.threadpool_limits(1):
        import oracle
        from mixed_precision_paged_amd import synth

        L = synth.mixed_batch_layer(li)
        c = L.paged
        H, D = c.num_kv_heads, c.head_dim
        nd = L.n_decode
        lens = c.seq_lens[:nd]
        ids, kv_start = routing_plan(L)
        dec, dec_lse = oracle.decode_attention(L.q_decode, c.k_target, c.v_target, c.k_compact, c.v_compact,
                                               c.v_scale, c.page_table[:nd], c.fidelity[:nd], lens, c.sm_scale)
        wk, wv = oracle.gather_compact_pages(c.k_compact, c.v_compact, c.v_scale, ids, True)
        rng = np.random.default_rng(seed)
        sample = []
        for i in range(len(L.prompt_lens)):
            sample += [int(L.cu_seqlens_q[i]) + r for r in sample_rows(int(L.prompt_lens[i]), rng)]
        sample = np.asarray(sample, dtype=np.int64)
        pw, plw = oracle.prefill_attention(L.q_prefill, wk.reshape(-1, H, D), wv.reshape(-1, H, D),
                                           L.cu_seqlens_q, kv_start, True, c.sm_scale, rows=sample)
        arrays = {
            "k_target": c.k_target, "v_target": c.v_target, "k_compact": c.k_compact,
            "v_compact": c.v_compact, "v_scale": c.v_scale, "page_table": c.page_table[:nd],
            "fidelity": c.fidelity[:nd], "seq_lens": lens, "q_decode": L.q_decode, "q_prefill": L.q_prefill,
            "cu_seqlens_q": L.cu_seqlens_q, "ids": ids, "kv_start": kv_start, "ws_k": wk, "ws_v": wv,
        }
        layout, off = {}, 0
        for name, a in arrays.items():
            a = np.ascontiguousarray(a)
            layout[name] = (off, a.dtype.str, a.shape)
            off += (a.nbytes + 255) // 256 * 256
        path = os.path.join(spool, f"layer{li:02d}.bin")
        mm = np.memmap(path, dtype=np.uint8, mode="w+", shape=(max(off, 1),))
        for name, a in arrays.items():
            o, _, _ = layout[name]
            a = np.ascontiguousarray(a)
            mm[o:o + a.nbytes] = a.reshape(-1).view(np.uint8)
        mm.flush()
        del mm
        expect = dict(dec=dec, dec_lse=dec_lse, sample=sample, pre=pw[sample], pre_lse=plw[sample],
                      n_decode=nd, max_len=int(lens.max()), prompt_len=int(L.prompt_lens.max()),
                      sm_scale=c.sm_scale, heads=(c.num_q_heads, H, D))
        return path, layout, expect


def load_layer(path: str, layout: dict) -> dict:
    """Main process: the layer's arrays as copy-on-write views of its file."""
    mm = np.memmap(path, dtype=np.uint8, mode="c")
    out = {}
    for name, (off, dt, shape) in layout.items():
        dt = np.dtype(dt)
        n = int(np.prod(shape)) if len(shape) else 1
        out[name] = mm[off:off + n * dt.itemsize].view(dt).reshape(shape)
    return out

"""Paged KV lookup: logical token -> (page, slot) -> physical page of one pool.

[ekv] section 2.1 (paged KV cache management): a request's logical blocks
map to physical blocks through a block table, and attention follows that
mapping in logical token order.  [ekv] section 3.2 and appendix B.3: each
page has a fidelity mode and pages of both modes are read in one batch.
[asym] "What changes in vLLM's prefill routing?": NHD layout, page size 16,
FP16 keys, E4M3 values, value scales applied in attention.

Readings taken where the pages are silent: the fidelity flag is one uint8 per
page-table entry (0 = TARGET, 1 = COMPACT, 2 = ElasticKV BASE); the page id
indexes the pool the flag selects (a BASE id b names half b % 2 of TARGET
block b // 2, see ``base.py``); the value scale is fp32 per (compact page, KV
head); token t of sequence b lives in logical page t // 16, slot t % 16; only
t < len_b is read.
"""
import numpy as np

from .base import base_page, base_values
from .e4m3 import decode_e4m3fn

PAGE = 16
TARGET = 0
COMPACT = 1
BASE = 2


def sequence_kv(k_target, v_target, k_compact, v_compact, v_scale,
                page_table_row, fidelity_row, seq_len):
    """Keys and values of one sequence in logical order, as float64.

    Returns K, V of shape [seq_len, Hkv, D].  Compact values are the exact
    products e4m3(byte) * scale (exact in float64: 4 x 24 significant bits).
    """
    seq_len = int(seq_len)
    pools = k_target if k_target is not None and k_target.size else k_compact
    hkv, d = pools.shape[2], pools.shape[3]
    K = np.empty((seq_len, hkv, d), dtype=np.float64)
    V = np.empty((seq_len, hkv, d), dtype=np.float64)
    for t in range(0, seq_len, PAGE):
        j = t // PAGE
        n = min(PAGE, seq_len - t)
        phys = int(page_table_row[j])
        flag = int(fidelity_row[j])
        if flag == TARGET:
            K[t:t + n] = k_target[phys, :n].astype(np.float64)
            V[t:t + n] = v_target[phys, :n].astype(np.float64)
        elif flag == COMPACT:
            K[t:t + n] = k_compact[phys, :n].astype(np.float64)
            V[t:t + n] = decode_e4m3fn(v_compact[phys, :n]) * \
                v_scale[phys].astype(np.float64)[None, :, None]
        elif flag == BASE:   # [ekv] BASE page phys: half phys % 2 of TARGET block phys // 2
            K[t:t + n] = base_values(base_page(k_target, phys)[:n])
            V[t:t + n] = base_values(base_page(v_target, phys)[:n])
        else:
            raise ValueError(f"fidelity flag {flag} is neither TARGET nor COMPACT")
    return K, V

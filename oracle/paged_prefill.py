"""Causal prefill read straight from mixed-fidelity pages (no workspace).

[asym] "Existing fallback: mixed-type prefill" and "What changes in vLLM's
prefill routing?": a prefill kernel can read the stored K16/V8 pages of a
fresh prompt directly instead of gathering them into an FP16 workspace.
[ekv] section 3.2: TARGET and compact pages of one sequence are read through
one page table, each in its own format.

Reading taken here: the direct route computes the same values the gather
route feeds to its FP16 prefill.  The keys and values of prompt p are its
tokens 0..L_p-1 in logical order (page t // 16, slot t % 16 of page-table row
p); a TARGET page contributes its FP16 K and V as stored; a compact page its
FP16 K and V = fp16(fp32(e4m3(byte)) * fp32(scale)) — the scaled gather's
rounding.  Attention is then the plain definition over those rows.
"""
import numpy as np

from .attention import prefill_attention
from .gather import gather_compact_pages

PAGE = 16
TARGET = 0
COMPACT = 1


def prompt_rows(k_target, v_target, k_compact, v_compact, v_scale, page_table_row,
                fidelity_row, length):
    """FP16 K and V rows [length, Hkv, D] of one prompt, as the direct route reads them."""
    pool = k_target if k_target is not None and np.size(k_target) else k_compact
    hkv, d = pool.shape[2], pool.shape[3]
    K = np.empty((length, hkv, d), dtype=np.float16)
    V = np.empty((length, hkv, d), dtype=np.float16)
    for t in range(0, length, PAGE):
        j = t // PAGE
        n = min(PAGE, length - t)
        phys = int(page_table_row[j])
        flag = int(fidelity_row[j])
        if flag == TARGET:
            K[t:t + n] = k_target[phys, :n]
            V[t:t + n] = v_target[phys, :n]
        elif flag == COMPACT:
            wk, wv = gather_compact_pages(k_compact, v_compact, v_scale, [phys], True)
            K[t:t + n] = wk[0, :n]
            V[t:t + n] = wv[0, :n]
        else:
            raise ValueError(f"fidelity flag {flag} is neither TARGET nor COMPACT")
    return K, V


def paged_prefill_attention(q, k_target, v_target, k_compact, v_compact, v_scale, page_table,
                            fidelity, cu_seqlens_q, causal, sm_scale, rows=None):
    """Attention of packed prompts (q [T, Hq, D], prompt p = rows cu[p]..cu[p+1]-1) over
    their own pages.  Returns out [T, Hq, D] float64 and lse [T, Hq]."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    ks, vs = [], []
    for p in range(cu.shape[0] - 1):
        L = int(cu[p + 1] - cu[p])
        K, V = prompt_rows(k_target, v_target, k_compact, v_compact, v_scale, page_table[p],
                           fidelity[p], L)
        ks.append(K)
        vs.append(V)
    k = np.concatenate(ks) if ks else np.zeros((0, 1, 1), np.float16)
    v = np.concatenate(vs) if vs else np.zeros((0, 1, 1), np.float16)
    return prefill_attention(q, k, v, cu, cu[:-1], causal, sm_scale, rows=rows)

"""Test-local construction of paged pools FROM contiguous per-sequence tensors.

This is the inverse direction of a paged lookup (a scatter into shuffled
physical pages), written independently of the oracle, so that comparing the
oracle's paged attention against a library routine on the contiguous tensors
checks the oracle's page/slot indexing and pool selection.
"""
import numpy as np

PAGE = 16


def build_paged(rng, keys, values16, codes, scales, fidelity_per_page, extra_pages=3):
    """keys[b]: fp16 [len_b, H, D]; values16[b]: fp16 [len_b, H, D] (TARGET data);
    codes[b]: uint8 [len_b, H, D] and scales[b]: fp32 [pages_b, H] (COMPACT data);
    fidelity_per_page[b]: list of 0/1 per logical page.
    Returns dict of pools + tables (unused slots filled with NaN / 0x7F)."""
    B = len(keys)
    H, D = keys[0].shape[1], keys[0].shape[2]
    lens = [k.shape[0] for k in keys]
    pages = [(n + PAGE - 1) // PAGE for n in lens]
    max_pages = max(1, max(pages))
    n_t = sum(sum(1 for f in fidelity_per_page[b] if f == 0) for b in range(B))
    n_c = sum(sum(1 for f in fidelity_per_page[b] if f == 1) for b in range(B))
    P_T, P_C = n_t + extra_pages, n_c + extra_pages
    kt = np.full((P_T, PAGE, H, D), np.nan, dtype=np.float16)
    vt = np.full((P_T, PAGE, H, D), np.nan, dtype=np.float16)
    kc = np.full((P_C, PAGE, H, D), np.nan, dtype=np.float16)
    vc = np.full((P_C, PAGE, H, D), 0x7F, dtype=np.uint8)
    sc = np.full((P_C, H), np.nan, dtype=np.float32)
    free_t = list(rng.permutation(P_T))
    free_c = list(rng.permutation(P_C))
    table = np.zeros((B, max_pages), dtype=np.int32)
    flags = np.zeros((B, max_pages), dtype=np.uint8)
    for b in range(B):
        for j in range(pages[b]):
            f = fidelity_per_page[b][j]
            lo, hi = j * PAGE, min(lens[b], (j + 1) * PAGE)
            if f == 0:
                phys = int(free_t.pop())
                for t in range(lo, hi):
                    kt[phys, t - lo] = keys[b][t]
                    vt[phys, t - lo] = values16[b][t]
            else:
                phys = int(free_c.pop())
                for t in range(lo, hi):
                    kc[phys, t - lo] = keys[b][t]
                    vc[phys, t - lo] = codes[b][t]
                sc[phys] = scales[b][j]
            table[b, j] = phys
            flags[b, j] = f
    return dict(k_target=kt, v_target=vt, k_compact=kc, v_compact=vc, v_scale=sc,
                page_table=table, fidelity=flags, seq_lens=np.array(lens, dtype=np.int32))

"""Algorithmic bytes and FLOPs of the hot path (what the method must move).

Per-pair byte model from the asymmetric-KV page ("Memory-Traffic Saturation
in Autoregressive Transformer Decode", table "Conventional equally sized K/V
tensors; raw payload ratios only"): K16/V16 = 4 bytes per K/V element pair,
K16/V8 = 3, K8/V8 = 2.  Its worked example (section "A bandwidth example with
explicit assumptions") and its slot count ("Physical storage" row of the
dense FP16 transfer table) pin the helpers below; see
``tests/golden/asym_byte_model.json``.

These counts are the roofline numerators: implementation traffic (split-K
partials, re-reads) is deliberately not counted.
"""
from __future__ import annotations

import numpy as np

PAGE = 16
BYTES_PER_PAIR = {"K16/V16": 4, "K16/V8": 3, "K8/V8": 2}


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, layout: str = "K16/V16") -> int:
    return layers * kv_heads * head_dim * BYTES_PER_PAIR[layout]


def kv_payload_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, layout: str) -> int:
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim, layout)


def reread_gbps(payload_bytes: float, seconds: float) -> float:
    """Decimal GB/s to move ``payload_bytes`` once in ``seconds``."""
    return payload_bytes / seconds / 1e9


def token_slots(pool_bytes: int, layers: int, kv_heads: int, head_dim: int, layout: str) -> int:
    """Whole token slots per layer a K/V byte pool holds."""
    return pool_bytes // kv_bytes_per_token(layers, kv_heads, head_dim, layout)


def decode_bytes(seq_lens, fidelity, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 out_bytes: int = 2, lse: bool = False, flags_read: bool = True,
                 bounds_read: bool = False) -> int:
    """Bytes one decode launch must move.

    K: 2 B per element for every valid token (1 B on an ElasticKV BASE page);
    V: 2 B (TARGET) or 1 B (COMPACT, BASE) per element; one fp32 scale per
    compact page per KV head; one int32 page id (and one uint8 flag when flags
    are read) per page; two int32 BASE bounds per sequence when the structured
    layout is read instead of flags; the FP16 query; the output (and fp32 LSE
    when requested).
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    fid = np.asarray(fidelity)
    HD = num_kv_heads * head_dim
    total = 0
    for b, n in enumerate(lens):
        pages = int((n + PAGE - 1) // PAGE)
        toks = np.minimum(PAGE, n - PAGE * np.arange(pages))
        kinds = fid[b, :pages].astype(np.int64)
        total += int((toks * np.where(kinds == 2, 1, 2)).sum()) * HD   # K16 or BASE K
        total += int((toks * np.where(kinds == 0, 2, 1)).sum()) * HD   # V16, V8 or BASE V
        total += int((kinds == 1).sum()) * num_kv_heads * 4        # scales
        total += pages * 4 + (pages if flags_read else 0)          # page ids, flags
    B = lens.shape[0]
    if bounds_read:
        total += B * 8                                             # BASE bounds
    total += B * num_q_heads * head_dim * 2                        # q
    total += B * num_q_heads * head_dim * out_bytes                # out
    if lse:
        total += B * num_q_heads * 4
    return total


def pack_bytes(n_pairs: int, num_kv_heads: int, head_dim: int):
    """(read, written) bytes of one ElasticKV pack launch: per pair two fp16 TARGET
    blocks of K and of V are read and one block of each is written, plus 3 int32 ids."""
    block = PAGE * num_kv_heads * head_dim * 2
    return n_pairs * (4 * block + 12), n_pairs * 2 * block


def gather_bytes(n_pages: int, num_kv_heads: int, head_dim: int):
    """(read, written) bytes of one gather of ``n_pages`` compact pages."""
    elems = n_pages * PAGE * num_kv_heads * head_dim
    read = elems * 3 + n_pages * num_kv_heads * 4 + n_pages * 4
    written = elems * 4
    return read, written


def quantize_bytes(n_valid, num_kv_heads: int, head_dim: int, n_valid_read: bool = True):
    """(read, written) bytes of one page-quantizer launch over pages holding ``n_valid``
    rows each: the valid rows' K16 + V16 (4 B per pair) and the per-page int32 entries
    (row start, destination id, row count) are read; whole pages of K16 + E4M3 V (3 B per
    pair, all 16 slots) and one fp32 scale per page and KV head are written."""
    n_valid = np.asarray(n_valid, dtype=np.int64)
    hd = num_kv_heads * head_dim
    n_pages = int(n_valid.size)
    read = int(n_valid.sum()) * hd * 4 + n_pages * (12 if n_valid_read else 8)
    written = n_pages * PAGE * hd * 3 + n_pages * num_kv_heads * 4
    return read, written


def append_bytes(n_tokens: int, num_kv_heads: int, head_dim: int):
    """(read, written) bytes of one TARGET append: K16 + V16 rows and one int32 slot each."""
    hd = num_kv_heads * head_dim
    return n_tokens * (hd * 4 + 4), n_tokens * hd * 4


def prefill_flops(prompt_lens, num_q_heads: int, head_dim: int, causal: bool = True) -> int:
    """Dense QK^T + PV FLOPs (masked-out pairs not counted)."""
    total = 0
    for L in np.asarray(prompt_lens, dtype=np.int64):
        pairs = L * (L + 1) // 2 if causal else L * L
        total += 2 * 2 * head_dim * num_q_heads * int(pairs)
    return total

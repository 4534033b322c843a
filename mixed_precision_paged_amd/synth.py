"""Seeded synthetic inputs for the mixed-fidelity paged-KV attention path.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It produces *stored* cache contents (page pools, page tables,
fidelity flags, value scales, queries) and holds none of the attention
arithmetic: no E4M3 decoding, no softmax, no gather.

Workload shapes follow the asymmetric-KV page ("Memory-Traffic Saturation in
Autoregressive Transformer Decode", section "What changes in vLLM's prefill
routing?"): NHD layout, 16-token pages, FP16 keys, FP8 E4M3 values with value
scales, 32 query / 8 KV heads, head dim 128.  The mixed-fidelity flag per page
follows the ElasticKV page ("Does Execution Require Target KV Fidelity?",
section 3.2, dual-mode attention): every logical page is either TARGET or a
compact page, and one batch mixes both.

Recipe (stated once, used everywhere):
  * values are N(0,1) drawn in float32 from numpy PCG64(seed), then rounded
    to FP16 (round-to-nearest-even); pools are drawn 256 pages at a time in
    the order K_target, V_target, K_compact, V_compact, then the queries;
  * optional outliers: each V element independently (probability
    ``outlier_frac``, drawn after the chunk's normals) is multiplied by
    ``outlier_mult`` before the FP16 cast;
  * compact pages store K as FP16 and V as E4M3FN bytes with one fp32 scale
    per (page, KV head) = fp32(absmax over the page's *valid* tokens x D of
    the FP16 V) / 448; an all-zero page gets scale 1.0.  The E4M3 encoding is
    the library cast ``torch.float8_e4m3fn`` (round-to-nearest-even) after
    clamping to +-448 (saturating);
  * exactly round(compact_frac * N) of the batch's logical pages are COMPACT,
    chosen uniformly; the rest are TARGET (FP16 K and V);
  * physical page ids come from seeded random permutations of each pool;
    pools carry unused slack pages;
  * every slot a sequence does not own (unused pool pages, slots past the
    sequence length in its last page) is poisoned with NaN (FP16 0x7E00,
    E4M3 0x7F, scale NaN) so a kernel that reads them shows it.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

PAGE_SIZE = 16
FP16_NAN_BITS = np.uint16(0x7E00)
E4M3_NAN_CODE = np.uint8(0x7F)
E4M3_MAX = 448.0

TARGET = 0
COMPACT = 1


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_fp16(x32: np.ndarray) -> np.ndarray:
    """float32 -> float16, round to nearest even (torch's multi-threaded CPU cast)."""
    import torch

    return torch.from_numpy(x32).to(torch.float16).numpy()


def normal_fp16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) drawn in float32, rounded to FP16."""
    return _to_fp16(rng.standard_normal(size=shape, dtype=np.float32))


def _values_with_outliers(rng, shape, outlier_frac, outlier_mult) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape, dtype=np.float32) < np.float32(outlier_frac)
        v[mask] *= np.float32(outlier_mult)
    return _to_fp16(v)


_CHUNK_PAGES = 256  # pages generated per draw (bounds host temporaries)


def _pool_fp16(rng, pages, H, D, outlier_frac, outlier_mult) -> np.ndarray:
    """fp16 [pages, 16, H, D] pool drawn chunk by chunk (normals, then outlier draws, per chunk)."""
    out = np.empty((pages, PAGE_SIZE, H, D), dtype=np.float16)
    for lo in range(0, pages, _CHUNK_PAGES):
        hi = min(pages, lo + _CHUNK_PAGES)
        out[lo:hi] = _values_with_outliers(rng, (hi - lo, PAGE_SIZE, H, D), outlier_frac, outlier_mult)
    return out


def quantize_pages_e4m3(v16: np.ndarray, valid_slots: np.ndarray):
    """Cache-writer stand-in: FP16 V pages -> (E4M3FN bytes, fp32 scale [P, Hkv]).

    v16: float16 [P, 16, Hkv, D]; valid_slots: int [P] tokens a page holds.
    Slots at or past ``valid_slots`` are ignored for the scale and poisoned.
    """
    import torch  # library casts (E4M3 encoding, fp16 -> fp32)

    P, S, H, D = v16.shape
    v32 = torch.from_numpy(v16).to(torch.float32)                       # exact
    slot_max = v32.abs().amax(dim=3)                                     # [P, 16, H]
    valid = torch.arange(S)[None, :] < torch.from_numpy(np.asarray(valid_slots))[:, None]  # [P, 16]
    absmax = torch.where(valid[:, :, None], slot_max, torch.zeros(())).amax(dim=1)  # [P, H]
    scale = absmax / np.float32(E4M3_MAX)                                # fp32 division
    scale = torch.where(absmax > 0, scale, torch.ones(()))
    scaled = (v32 / scale[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8)
    del scaled, v32
    codes[~valid] = int(E4M3_NAN_CODE)
    scale = scale.numpy().astype(np.float32)
    scale[np.asarray(valid_slots) <= 0] = np.float32(np.nan)
    return codes.numpy(), scale


def _poison_fp16(pool: np.ndarray, valid_slots: np.ndarray) -> None:
    bits = pool.view(np.uint16)
    slot = np.arange(pool.shape[1])[None, :]
    bad = slot >= valid_slots[:, None]  # [P, 16]
    bits[bad] = FP16_NAN_BITS


@dataclasses.dataclass
class PagedCase:
    """One batch of paged KV plus queries (all host numpy arrays)."""

    q: np.ndarray                 # fp16 [B, Hq, D] (decode) or [T, Hq, D] (prefill)
    k_target: np.ndarray          # fp16 [P_T, 16, Hkv, D]
    v_target: np.ndarray          # fp16 [P_T, 16, Hkv, D]
    k_compact: np.ndarray         # fp16 [P_C, 16, Hkv, D]
    v_compact: np.ndarray         # uint8 (E4M3FN) [P_C, 16, Hkv, D]
    v_scale: np.ndarray           # fp32 [P_C, Hkv]
    page_table: np.ndarray        # int32 [B, max_pages]
    fidelity: np.ndarray          # uint8 [B, max_pages], 0 = TARGET, 1 = COMPACT
    seq_lens: np.ndarray          # int32 [B]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sm_scale: float

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


def _pool_size(used: int, pool_pages: Optional[int], slack_frac: float) -> int:
    if pool_pages is not None:
        if pool_pages < used:
            raise ValueError(f"pool of {pool_pages} pages cannot hold {used}")
        return pool_pages
    return used + int(math.ceil(used * slack_frac))


def make_paged_case(
    seed: int,
    seq_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    compact_frac: float = 1.0,
    outlier_frac: float = 0.0,
    outlier_mult: float = 20.0,
    slack_frac: float = 0.0625,
    target_pool_pages: Optional[int] = None,
    compact_pool_pages: Optional[int] = None,
    query_rows: Optional[int] = None,
    compact_logical: Optional[np.ndarray] = None,
) -> PagedCase:
    """Build a paged batch.  ``query_rows`` defaults to one query per sequence.

    ``compact_logical`` (bool [B, max_pages]) overrides the random choice of
    COMPACT pages (used for the prefill route, whose pages are all compact).
    """
    rng = _rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B = lens.shape[0]
    n_pages = (lens + PAGE_SIZE - 1) // PAGE_SIZE
    max_pages = int(max(1, n_pages.max() if B else 1))
    owned = np.arange(max_pages)[None, :] < n_pages[:, None]  # logical pages that exist
    total = int(owned.sum())

    # which logical pages are compact
    if compact_logical is not None:
        is_compact = np.asarray(compact_logical, dtype=bool) & owned
    else:
        n_compact = int(round(compact_frac * total))
        flat = np.flatnonzero(owned.ravel())
        chosen = rng.choice(flat, size=n_compact, replace=False) if n_compact else np.empty(0, np.int64)
        is_compact = np.zeros(B * max_pages, dtype=bool)
        is_compact[chosen] = True
        is_compact = is_compact.reshape(B, max_pages)
    is_target = owned & ~is_compact
    n_c_used = int(is_compact.sum())
    n_t_used = int(is_target.sum())
    P_C = _pool_size(n_c_used, compact_pool_pages, slack_frac)
    P_T = _pool_size(n_t_used, target_pool_pages, slack_frac)

    page_table = np.zeros((B, max_pages), dtype=np.int32)
    fidelity = np.zeros((B, max_pages), dtype=np.uint8)
    perm_c = rng.permutation(P_C)[:n_c_used].astype(np.int32)
    perm_t = rng.permutation(P_T)[:n_t_used].astype(np.int32)
    page_table[is_compact] = perm_c
    page_table[is_target] = perm_t
    fidelity[is_compact] = COMPACT

    # tokens held by each physical page (0 for slack pages)
    slot_count = np.minimum(PAGE_SIZE, lens[:, None] - PAGE_SIZE * np.arange(max_pages)[None, :])
    valid_c = np.zeros(P_C, dtype=np.int64)
    valid_t = np.zeros(P_T, dtype=np.int64)
    valid_c[perm_c] = slot_count[is_compact]
    valid_t[perm_t] = slot_count[is_target]

    H, D = num_kv_heads, head_dim
    k_target = _pool_fp16(rng, P_T, H, D, 0.0, outlier_mult)
    v_target = _pool_fp16(rng, P_T, H, D, outlier_frac, outlier_mult)
    _poison_fp16(k_target, valid_t)
    _poison_fp16(v_target, valid_t)

    k_compact = _pool_fp16(rng, P_C, H, D, 0.0, outlier_mult)
    v_compact = np.empty((P_C, PAGE_SIZE, H, D), dtype=np.uint8)
    v_scale = np.empty((P_C, H), dtype=np.float32)
    for lo in range(0, P_C, _CHUNK_PAGES):
        hi = min(P_C, lo + _CHUNK_PAGES)
        v16 = _values_with_outliers(rng, (hi - lo, PAGE_SIZE, H, D), outlier_frac, outlier_mult)
        v_compact[lo:hi], v_scale[lo:hi] = quantize_pages_e4m3(v16, valid_c[lo:hi])
    _poison_fp16(k_compact, valid_c)

    rows = B if query_rows is None else query_rows
    q = normal_fp16(rng, (rows, num_q_heads, D))
    return PagedCase(
        q=q, k_target=k_target, v_target=v_target, k_compact=k_compact,
        v_compact=v_compact, v_scale=v_scale, page_table=page_table,
        fidelity=fidelity, seq_lens=lens.astype(np.int32),
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        sm_scale=1.0 / math.sqrt(head_dim),
    )


# ---------------------------------------------------------------- workloads
# The five workloads: sizes, seeds and structure.  Each returns host arrays.

def tiny_decode_case(seed: int = 1) -> PagedCase:
    """Two sequences (37, 64 tokens), 4 q / 1 KV head, D 64, all compact, 16-page pool."""
    return make_paged_case(seed, [37, 64], 4, 1, 64, compact_frac=1.0, compact_pool_pages=16)


def compact_decode_case(seed: int = 2, batch: int = 32, ctx: int = 8192) -> PagedCase:
    """Batch 32, context 8192, 32 q / 8 KV heads, D 128, all compact, pool 16,384 + 6.25%."""
    return make_paged_case(seed, [ctx] * batch, 32, 8, 128, compact_frac=1.0)


def mixed_decode_lens(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    return _rng(seed + 1_000_003).integers(lo, hi + 1, size=batch)


def mixed_decode_case(seed: int = 3, batch: int = 64, lo: int = 1024, hi: int = 16384) -> PagedCase:
    """Batch 64, contexts U[1024, 16384], 30% compact pages, 1% V outliers x20."""
    lens = mixed_decode_lens(seed, batch, lo, hi)
    return make_paged_case(seed, lens, 32, 8, 128, compact_frac=0.3,
                           outlier_frac=0.01, outlier_mult=20.0)


@dataclasses.dataclass
class PrefillCase:
    """Fresh prompts stored in compact pages, plus packed queries."""

    paged: PagedCase              # page_table rows = prompts; q = packed [T, Hq, D]
    prompt_lens: np.ndarray       # int32 [n]
    cu_seqlens_q: np.ndarray      # int32 [n + 1]

    def chunk_pages(self, prompts: Sequence[int]) -> tuple:
        """Page ids of the listed prompts (logical order) and each prompt's first workspace row."""
        ids: List[np.ndarray] = []
        kv_start = []
        row = 0
        for p in prompts:
            n = int((self.prompt_lens[p] + PAGE_SIZE - 1) // PAGE_SIZE)
            ids.append(self.paged.page_table[p, :n])
            kv_start.append(row)
            row += n * PAGE_SIZE
        return np.concatenate(ids).astype(np.int32), np.asarray(kv_start, dtype=np.int32)


def make_prefill_case(seed: int, prompt_lens: Sequence[int], num_q_heads: int,
                      num_kv_heads: int, head_dim: int,
                      compact_pool_pages: Optional[int] = None) -> PrefillCase:
    lens = np.asarray(prompt_lens, dtype=np.int64)
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    paged = make_paged_case(seed, lens, num_q_heads, num_kv_heads, head_dim,
                            compact_frac=1.0, compact_pool_pages=compact_pool_pages,
                            query_rows=int(cu[-1]))
    return PrefillCase(paged=paged, prompt_lens=lens.astype(np.int32), cu_seqlens_q=cu)


def compact_prefill_case(seed: int = 4, prompts: int = 32, length: int = 8192) -> PrefillCase:
    """32 fresh prompts x 8192 tokens, 32 q / 8 KV heads, D 128, pool 16,384 + 6.25%."""
    return make_prefill_case(seed, [length] * prompts, 32, 8, 128)


@dataclasses.dataclass
class MixedBatchLayer:
    """One layer of the mixed batch: decode rows first, then fresh-prefill rows."""

    paged: PagedCase              # rows 0..n_decode-1 = decode seqs, then prompts
    n_decode: int
    prompt_lens: np.ndarray
    q_decode: np.ndarray          # fp16 [n_decode, Hq, D]
    q_prefill: np.ndarray         # fp16 [sum(prompt_lens), Hq, D]
    cu_seqlens_q: np.ndarray      # int32 [n_prompts + 1]


def mixed_batch_layer(layer: int, n_decode: int = 32, lo: int = 4096, hi: int = 32768,
                      n_prompts: int = 4, prompt_len: int = 2048,
                      compact_frac: float = 0.3) -> MixedBatchLayer:
    """Per-layer inputs of the 36-layer mixed batch (seed 5000 + layer)."""
    seed = 5000 + layer
    dec_lens = mixed_decode_lens(seed, n_decode, lo, hi)
    lens = np.concatenate([dec_lens, np.full(n_prompts, prompt_len)])
    n_pages = (lens + PAGE_SIZE - 1) // PAGE_SIZE
    max_pages = int(n_pages.max())
    rng = _rng(seed + 7)
    # decode pages: exactly round(frac * N) compact; prompt pages: all compact
    owned = np.arange(max_pages)[None, :] < n_pages[:, None]
    dec_owned = owned.copy()
    dec_owned[n_decode:] = False
    flat = np.flatnonzero(dec_owned.ravel())
    n_c = int(round(compact_frac * flat.size))
    chosen = rng.choice(flat, size=n_c, replace=False)
    compact = np.zeros(owned.size, dtype=bool)
    compact[chosen] = True
    compact = compact.reshape(owned.shape)
    compact[n_decode:] = owned[n_decode:]
    T = n_prompts * prompt_len
    paged = make_paged_case(seed, lens, 32, 8, 128, compact_logical=compact,
                            query_rows=n_decode + T)
    cu = np.arange(n_prompts + 1, dtype=np.int32) * prompt_len
    return MixedBatchLayer(paged=paged, n_decode=n_decode,
                           prompt_lens=np.full(n_prompts, prompt_len, dtype=np.int32),
                           q_decode=paged.q[:n_decode], q_prefill=paged.q[n_decode:],
                           cu_seqlens_q=cu)


@dataclasses.dataclass
class WriterCase:
    """Fresh FP16 K/V rows of packed prompts, cut into pages for the cache writer."""

    k_rows: np.ndarray            # fp16 [T, Hkv, D]
    v_rows: np.ndarray            # fp16 [T, Hkv, D]
    prompt_lens: np.ndarray       # int32 [n]
    row_start: np.ndarray         # int32 [n_pages]: first row of each page
    n_valid: np.ndarray           # int32 [n_pages]: rows in each page (16, or fewer at a prompt's end)
    dst_pages: np.ndarray         # int32 [n_pages]: distinct compact-pool ids (seeded permutation)
    n_compact_pages: int          # pool size: pages + 6.25% slack
    num_kv_heads: int
    head_dim: int


def make_writer_case(seed: int, prompt_lens: Sequence[int], num_kv_heads: int, head_dim: int,
                     outlier_frac: float = 0.0, outlier_mult: float = 1.0,
                     slack_frac: float = 0.0625) -> WriterCase:
    """K then V rows drawn like pool pages (256 pages of rows at a time), trimmed to the
    prompts' total length; then the pool permutation for the destination ids."""
    rng = _rng(seed)
    lens = np.asarray(prompt_lens, dtype=np.int64)
    T = int(lens.sum())
    row_pages = (T + PAGE_SIZE - 1) // PAGE_SIZE
    k = _pool_fp16(rng, row_pages, num_kv_heads, head_dim, 0.0, 1.0)
    k = k.reshape(-1, num_kv_heads, head_dim)[:T]
    v = _pool_fp16(rng, row_pages, num_kv_heads, head_dim, outlier_frac, outlier_mult)
    v = v.reshape(-1, num_kv_heads, head_dim)[:T]
    starts, valid = [], []
    row = 0
    for n in lens:
        j = np.arange((int(n) + PAGE_SIZE - 1) // PAGE_SIZE)
        starts.append(row + PAGE_SIZE * j)
        valid.append(np.minimum(PAGE_SIZE, int(n) - PAGE_SIZE * j))
        row += int(n)
    row_start = np.concatenate(starts).astype(np.int32) if starts else np.zeros(0, np.int32)
    n_valid = np.concatenate(valid).astype(np.int32) if valid else np.zeros(0, np.int32)
    n_pool = _pool_size(row_start.size, None, slack_frac)
    dst = rng.permutation(n_pool)[:row_start.size].astype(np.int32)
    return WriterCase(k_rows=k, v_rows=v, prompt_lens=lens.astype(np.int32), row_start=row_start,
                      n_valid=n_valid, dst_pages=dst, n_compact_pages=n_pool,
                      num_kv_heads=num_kv_heads, head_dim=head_dim)


def writer_prefill_case(seed: int = 4, prompts: int = 32, length: int = 8192) -> WriterCase:
    """The compact-prefill prompt set (32 x 8192 tokens, 8 KV heads, D 128) written
    into 16,384 compact pages of a 17,408-page pool."""
    return make_writer_case(seed, [length] * prompts, 8, 128)


BASE = 2


@dataclasses.dataclass
class ElasticCase:
    """A paged batch in which some logical page pairs are ElasticKV BASE pages."""

    paged: PagedCase              # fidelity 0 / 1 / 2; a BASE id b = half b % 2 of TARGET block b // 2
    base_bounds: np.ndarray       # int32 [B, 2]: BASE logical pages [lo, hi) (structured layouts)
    structured: bool              # True: every sequence is TARGET-BASE-TARGET within base_bounds


def make_elastic_case(seed: int, seq_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                      head_dim: int, sink_pages: int = 2, recent_pages: int = 32,
                      structured: bool = True, base_pair_frac: float = 0.5,
                      compact_frac: float = 0.0) -> ElasticCase:
    """Start from a seeded paged batch (TARGET pages, plus compact ones if compact_frac > 0)
    and demote logical pairs (2i, 2i+1) of full TARGET pages outside the protected sink
    (first ``sink_pages``) and recent (last ``recent_pages``) pages: all of them when
    ``structured`` (one BASE range per sequence), else each with probability
    ``base_pair_frac``.  A demoted pair is stored as in a demotion packed in place: the
    first page's TARGET block holds the high bytes of both pages (first half, second half)
    and the second page's block is freed (filled with NaN, never read)."""
    c = make_paged_case(seed, seq_lens, num_q_heads, num_kv_heads, head_dim,
                        compact_frac=compact_frac)
    rng = _rng(seed + 1)
    lens = c.seq_lens.astype(np.int64)
    B = lens.shape[0]
    full = lens // PAGE_SIZE                       # full pages per sequence
    bounds = np.zeros((B, 2), dtype=np.int32)
    k_bytes = c.k_target.view(np.uint8).reshape(c.k_target.shape[0], 2, PAGE_SIZE, num_kv_heads, head_dim)
    v_bytes = c.v_target.view(np.uint8).reshape(c.v_target.shape[0], 2, PAGE_SIZE, num_kv_heads, head_dim)
    for b in range(B):
        lo = (sink_pages + 1) // 2 * 2
        hi = max(lo, (min(int(full[b]), int((lens[b] + PAGE_SIZE - 1) // PAGE_SIZE) - recent_pages)) // 2 * 2)
        pairs = []
        for j in range(lo, hi, 2):
            if c.fidelity[b, j] != TARGET or c.fidelity[b, j + 1] != TARGET:
                continue
            if structured or rng.random() < base_pair_frac:
                pairs.append(j)
        if structured:
            bounds[b] = (lo, hi) if pairs else (0, 0)
        for j in pairs:
            pa, pb = int(c.page_table[b, j]), int(c.page_table[b, j + 1])
            hk = (c.k_target[pa].view(np.uint16) >> 8).astype(np.uint8), (c.k_target[pb].view(np.uint16) >> 8).astype(np.uint8)
            hv = (c.v_target[pa].view(np.uint16) >> 8).astype(np.uint8), (c.v_target[pb].view(np.uint16) >> 8).astype(np.uint8)
            k_bytes[pa, 0], k_bytes[pa, 1] = hk
            v_bytes[pa, 0], v_bytes[pa, 1] = hv
            c.k_target[pb].view(np.uint16)[...] = FP16_NAN_BITS
            c.v_target[pb].view(np.uint16)[...] = FP16_NAN_BITS
            c.page_table[b, j], c.page_table[b, j + 1] = 2 * pa, 2 * pa + 1
            c.fidelity[b, j] = c.fidelity[b, j + 1] = BASE
    return ElasticCase(paged=c, base_bounds=bounds, structured=structured)


def elastic_decode_case(seed: int = 6, batch: int = 32, ctx: int = 8192) -> ElasticCase:
    """B 32, context 8192, 32 q / 8 KV heads, D 128: TARGET attention-sink pair and recent
    512 tokens, the middle 478 pages (239 pairs) BASE, structured layout."""
    return make_elastic_case(seed, [ctx] * batch, 32, 8, 128, sink_pages=2, recent_pages=32)

"""Python binding of libekv.so (C ABI in include/ekv.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, statuses become exceptions.  Every step of the
computation runs in the HIP kernels of libekv.so; there is no fallback.
Importing this module raises ImportError if the library has not been built
(``python -m mixed_precision_paged_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libekv.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mixed_precision_paged_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

PAGE_SIZE = 16
FIDELITY_TARGET = 0
FIDELITY_COMPACT = 1
FIDELITY_BASE = 2
MAX_PREFILL_TOKENS = 8192
DECODE_BALANCED = -1  # pages_per_split: equal shares of all page-heads per workgroup
NOALLOC_SCRATCH_BYTES = 8 << 20  # static scratch of ekv_decode_attention_noalloc

EKV_OK = 0
EKV_ERR_INVALID_ARG = 1
EKV_ERR_UNSUPPORTED = 2
EKV_ERR_WORKSPACE_TOO_SMALL = 3
EKV_ERR_NOT_ELIGIBLE = 4
EKV_ERR_HIP = 5
EKV_F16 = 0
EKV_F32 = 1

EXPORTED = (
    "ekv_abi_version", "ekv_status_string", "ekv_last_error", "ekv_decode_pages_per_split",
    "ekv_decode_plan_pages_per_split", "ekv_decode_scratch_bytes", "ekv_decode_attention",
    "ekv_decode_attention_elastic", "ekv_gather_compact_pages", "ekv_prefill_attention",
    "ekv_prefill_paged_attention", "ekv_append_tokens", "ekv_quantize_pages", "ekv_pack_base_pairs",
    "ekv_e4m3_to_f16", "ekv_decode_attention_noalloc", "ekv_build_id",
)


class PagedKV(ctypes.Structure):
    _fields_ = [
        ("k_target", ctypes.c_void_p), ("v_target", ctypes.c_void_p), ("n_target_pages", ctypes.c_int32),
        ("k_compact", ctypes.c_void_p), ("v_compact", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("n_compact_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
    ]


_i32, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_lib.ekv_abi_version.restype = _i32
_lib.ekv_build_id.restype = ctypes.c_char_p
_lib.ekv_status_string.restype = ctypes.c_char_p
_lib.ekv_status_string.argtypes = [ctypes.c_int]
_lib.ekv_last_error.restype = ctypes.c_char_p
_lib.ekv_decode_pages_per_split.restype = _i32
_lib.ekv_decode_pages_per_split.argtypes = [_i32, _i32, _i32]
_lib.ekv_decode_plan_pages_per_split.restype = _i32
_lib.ekv_decode_plan_pages_per_split.argtypes = [_vp, _i32, _i32]
_lib.ekv_decode_scratch_bytes.restype = _sz
_lib.ekv_decode_scratch_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.ekv_decode_attention.restype = ctypes.c_int
_lib.ekv_decode_attention.argtypes = [
    ctypes.POINTER(PagedKV), _vp, _i32, _i32, _vp, _i32, _vp, _vp, _i32, _f32, _vp, ctypes.c_int,
    _vp, _i32, _vp, _sz, _vp]
_lib.ekv_decode_attention_noalloc.restype = ctypes.c_int
_lib.ekv_decode_attention_noalloc.argtypes = [
    ctypes.POINTER(PagedKV), _vp, _i32, _i32, _vp, _i32, _vp, _vp, _i32, _f32, _vp, ctypes.c_int,
    _vp, _i32, _vp]
_lib.ekv_decode_attention_elastic.restype = ctypes.c_int
_lib.ekv_decode_attention_elastic.argtypes = [
    ctypes.POINTER(PagedKV), _vp, _i32, _i32, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _f32, _vp,
    ctypes.c_int, _vp, _i32, _vp, _sz, _vp]
_lib.ekv_pack_base_pairs.restype = ctypes.c_int
_lib.ekv_pack_base_pairs.argtypes = [ctypes.POINTER(PagedKV), _vp, _vp, _vp, _i32, _vp]
_lib.ekv_gather_compact_pages.restype = ctypes.c_int
_lib.ekv_gather_compact_pages.argtypes = [ctypes.POINTER(PagedKV), _vp, _i32, _i32, _vp, _vp, _i32, _vp]
_lib.ekv_prefill_attention.restype = ctypes.c_int
_lib.ekv_prefill_attention.argtypes = [
    _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, ctypes.c_int,
    _vp, _vp]
_lib.ekv_prefill_paged_attention.restype = ctypes.c_int
_lib.ekv_prefill_paged_attention.argtypes = [
    ctypes.POINTER(PagedKV), _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _f32, _vp,
    ctypes.c_int, _vp, _vp]
_lib.ekv_append_tokens.restype = ctypes.c_int
_lib.ekv_append_tokens.argtypes = [ctypes.POINTER(PagedKV), _vp, _vp, _vp, _i32, _vp]
_lib.ekv_quantize_pages.restype = ctypes.c_int
_lib.ekv_quantize_pages.argtypes = [ctypes.POINTER(PagedKV), _vp, _vp, ctypes.c_int64, _vp, _vp, _vp,
                                    _i32, _vp]
_lib.ekv_e4m3_to_f16.restype = ctypes.c_int
_lib.ekv_e4m3_to_f16.argtypes = [_vp, _i32, _vp, _i32, _i32, _vp]


class EkvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{ekv_status_string(status)} ({status}): {detail}")


def ekv_abi_version() -> int:
    return int(_lib.ekv_abi_version())


def ekv_build_id() -> str:
    return _lib.ekv_build_id().decode()


def ekv_status_string(status: int) -> str:
    return _lib.ekv_status_string(int(status)).decode()


def ekv_last_error() -> str:
    return _lib.ekv_last_error().decode()


def _check(status: int) -> None:
    if status != EKV_OK:
        raise EkvError(status, ekv_last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libekv must be contiguous")
    return t.data_ptr() or None


_F16, _F32, _I32, _U8 = torch.float16, torch.float32, torch.int32, torch.uint8


def _arg(t: Optional[torch.Tensor], name: str, dtypes=None) -> Optional[int]:
    """Device pointer of a contiguous GPU tensor of an expected dtype (None passes through):
    a host tensor would hand the kernels a host address."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor, got one on {t.device}")
    if dtypes is not None:
        dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
        if t.dtype not in dtypes:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    return _ptr(t)


def _same_shape(a: Optional[torch.Tensor], b: Optional[torch.Tensor], what: str) -> None:
    if a is not None and b is not None and tuple(a.shape) != tuple(b.shape):
        raise ValueError(f"{what}: shapes {tuple(a.shape)} and {tuple(b.shape)} differ")


def _expect(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_decode_shapes(kv: PagedKV, q, page_table, seq_lens, out, lse, rows_of=None) -> None:
    """Shapes the decode entry points assume, checked before any launch."""
    _expect(q.dim() == 3, f"q must be [batch, num_q_heads, head_dim], got {tuple(q.shape)}")
    batch, hq, d = q.shape
    _expect(d == kv.head_dim, f"q has head dim {d}, the pools {kv.head_dim}")
    _expect(page_table.dim() == 2 and int(page_table.shape[0]) == batch,
            f"page_table must have one row per sequence ({batch}), got {tuple(page_table.shape)}")
    _expect(tuple(seq_lens.shape) == (batch,), f"seq_lens must be [{batch}], got {tuple(seq_lens.shape)}")
    _expect(tuple(out.shape) == tuple(q.shape), f"out must be {tuple(q.shape)}, got {tuple(out.shape)}")
    _expect(lse is None or tuple(lse.shape) == (batch, hq), f"lse must be [{batch}, {hq}], got "
            f"{None if lse is None else tuple(lse.shape)}")


def _check_prefill_out(q, out, lse) -> None:
    _expect(tuple(out.shape) == tuple(q.shape), f"out must be {tuple(q.shape)}, got {tuple(out.shape)}")
    _expect(lse is None or tuple(lse.shape) == tuple(q.shape[:2]),
            f"lse must be {tuple(q.shape[:2])}, got {None if lse is None else tuple(lse.shape)}")


def _kv_ref(kv: PagedKV):
    """The descriptor for the call, after checking that its pools live on the GPU."""
    for t in getattr(kv, "_tensors", ()):
        if t is not None and not t.is_cuda:
            raise ValueError(f"page pools must be device tensors, got one on {t.device}")
    return ctypes.byref(kv)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return EKV_F16
    if t.dtype == torch.float32:
        return EKV_F32
    raise TypeError(f"output dtype {t.dtype} is not float16/float32")


def paged_kv(num_kv_heads: int, head_dim: int, k_target=None, v_target=None, k_compact=None,
             v_compact=None, v_scale=None) -> PagedKV:
    """Descriptor of one layer's page pools.  The descriptor holds references to the
    tensors whose device pointers it carries, so they live at least as long as it does."""
    n_t = int(k_target.shape[0]) if k_target is not None else 0
    n_c = int(k_compact.shape[0]) if k_compact is not None else 0
    for t, dt in ((k_target, torch.float16), (v_target, torch.float16), (k_compact, torch.float16),
                  (v_compact, torch.uint8), (v_scale, torch.float32)):
        if t is not None and t.dtype != dt:
            raise TypeError(f"pool tensor has dtype {t.dtype}, expected {dt}")
    desc = PagedKV(_ptr(k_target), _ptr(v_target), n_t, _ptr(k_compact), _ptr(v_compact),
                   _ptr(v_scale), n_c, num_kv_heads, head_dim, PAGE_SIZE)
    desc._tensors = (k_target, v_target, k_compact, v_compact, v_scale)
    return desc


def ekv_decode_pages_per_split(batch: int, num_kv_heads: int, max_seq_len: int) -> int:
    return int(_lib.ekv_decode_pages_per_split(batch, num_kv_heads, max_seq_len))


def ekv_decode_plan_pages_per_split(seq_lens_host, num_kv_heads: int) -> int:
    """Split plan from host-side lengths (a numpy int32 array or sequence)."""
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    return int(_lib.ekv_decode_plan_pages_per_split(lens.ctypes.data if lens.size else None,
                                                    int(lens.size), int(num_kv_heads)))


def ekv_decode_scratch_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             max_seq_len: int, pages_per_split: int = 0) -> int:
    return int(_lib.ekv_decode_scratch_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                             max_seq_len, pages_per_split))


def ekv_decode_attention(kv: PagedKV, q: torch.Tensor, page_table: torch.Tensor,
                         fidelity: Optional[torch.Tensor], seq_lens: torch.Tensor, max_seq_len: int,
                         sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                         scratch: Optional[torch.Tensor] = None, pages_per_split: int = 0,
                         stream=None) -> None:
    """GQA decode over paged TARGET/compact KV (see ekv.h).  Writes ``out`` (and ``lse``)."""
    _check_decode_shapes(kv, q, page_table, seq_lens, out, lse)
    batch, hq, _ = q.shape
    _same_shape(page_table, fidelity, "page_table and fidelity")
    if scratch is None:
        need = ekv_decode_scratch_bytes(batch, hq, kv.num_kv_heads, kv.head_dim, max_seq_len,
                                        pages_per_split)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(_lib.ekv_decode_attention(
        _kv_ref(kv), _arg(q, "q", _F16), batch, hq, _arg(page_table, "page_table", _I32),
        int(page_table.shape[1]), _arg(fidelity, "fidelity", _U8), _arg(seq_lens, "seq_lens", _I32),
        int(max_seq_len), float(sm_scale), _arg(out, "out"), _dtype_code(out), _arg(lse, "lse", _F32),
        int(pages_per_split), _arg(scratch, "scratch"), scratch.numel() * scratch.element_size(),
        _stream(stream)))


def ekv_decode_attention_noalloc(kv: PagedKV, q: torch.Tensor, page_table: torch.Tensor,
                                 fidelity: Optional[torch.Tensor], seq_lens: torch.Tensor, max_seq_len: int,
                                 sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                                 pages_per_split: int = 0, stream=None) -> None:
    """ekv_decode_attention with the library's static scratch: allocates nothing (see ekv.h)."""
    _check_decode_shapes(kv, q, page_table, seq_lens, out, lse)
    batch, hq, _ = q.shape
    _same_shape(page_table, fidelity, "page_table and fidelity")
    _check(_lib.ekv_decode_attention_noalloc(
        _kv_ref(kv), _arg(q, "q", _F16), batch, hq, _arg(page_table, "page_table", _I32),
        int(page_table.shape[1]), _arg(fidelity, "fidelity", _U8), _arg(seq_lens, "seq_lens", _I32),
        int(max_seq_len), float(sm_scale), _arg(out, "out"), _dtype_code(out), _arg(lse, "lse", _F32),
        int(pages_per_split), _stream(stream)))


def ekv_decode_attention_elastic(kv: PagedKV, q: torch.Tensor, page_table: torch.Tensor,
                                 fidelity: Optional[torch.Tensor], base_bounds: Optional[torch.Tensor],
                                 has_base: bool, seq_lens: torch.Tensor, max_seq_len: int,
                                 sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                                 scratch: Optional[torch.Tensor] = None, pages_per_split: int = 0,
                                 stream=None) -> None:
    """Decode over TARGET / compact / ElasticKV BASE pages (see ekv.h): per-page flags
    (0, 1, 2) or per-sequence BASE bounds [B, 2] for TARGET-BASE-TARGET layouts."""
    _check_decode_shapes(kv, q, page_table, seq_lens, out, lse)
    batch, hq, _ = q.shape
    _expect(base_bounds is None or tuple(base_bounds.shape) == (batch, 2),
            f"base_bounds must be [{batch}, 2], got {None if base_bounds is None else tuple(base_bounds.shape)}")
    _same_shape(page_table, fidelity, "page_table and fidelity")
    if scratch is None:
        need = ekv_decode_scratch_bytes(batch, hq, kv.num_kv_heads, kv.head_dim, max_seq_len,
                                        pages_per_split)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(_lib.ekv_decode_attention_elastic(
        _kv_ref(kv), _arg(q, "q", _F16), batch, hq, _arg(page_table, "page_table", _I32),
        int(page_table.shape[1]), _arg(fidelity, "fidelity", _U8), _arg(base_bounds, "base_bounds", _I32),
        1 if has_base else 0, _arg(seq_lens, "seq_lens", _I32), int(max_seq_len), float(sm_scale),
        _arg(out, "out"), _dtype_code(out), _arg(lse, "lse", _F32), int(pages_per_split),
        _arg(scratch, "scratch"), scratch.numel() * scratch.element_size(), _stream(stream)))


def ekv_pack_base_pairs(kv: PagedKV, src_a: torch.Tensor, src_b: torch.Tensor, dst: torch.Tensor,
                        stream=None) -> None:
    """Pack TARGET block pairs into BASE blocks in the TARGET pools (see ekv.h)."""
    _same_shape(src_a, dst, "src_a and dst")
    _same_shape(src_b, dst, "src_b and dst")
    _check(_lib.ekv_pack_base_pairs(_kv_ref(kv), _arg(src_a, "src_a", _I32), _arg(src_b, "src_b", _I32),
                                    _arg(dst, "dst", _I32), int(dst.shape[0]), _stream(stream)))


def ekv_gather_compact_pages(kv: PagedKV, page_ids: torch.Tensor, apply_scale: bool,
                             ws_k: torch.Tensor, ws_v: torch.Tensor, n_pages: Optional[int] = None,
                             stream=None) -> None:
    """Gather compact pages into the FP16 workspace (see ekv.h).

    ws_k, ws_v: [capacity, 16, Hkv, D] fp16 (the capacity is their first dimension)."""
    page = (PAGE_SIZE, kv.num_kv_heads, kv.head_dim)
    for name, ws in (("ws_k", ws_k), ("ws_v", ws_v)):
        _expect(ws.dim() == 4 and tuple(ws.shape[1:]) == page,
                f"{name} must be [capacity, {', '.join(map(str, page))}], got {tuple(ws.shape)}")
    _expect(page_ids.dim() == 1, f"page_ids must be one-dimensional, got {tuple(page_ids.shape)}")
    n = int(page_ids.shape[0]) if n_pages is None else int(n_pages)
    if n > int(page_ids.shape[0]):
        raise ValueError(f"n_pages {n} exceeds the {int(page_ids.shape[0])} page ids given")
    _same_shape(ws_k, ws_v, "ws_k and ws_v")
    _check(_lib.ekv_gather_compact_pages(
        _kv_ref(kv), _arg(page_ids, "page_ids", _I32), n, 1 if apply_scale else 0,
        _arg(ws_k, "ws_k", _F16), _arg(ws_v, "ws_v", _F16), int(ws_k.shape[0]), _stream(stream)))


def ekv_prefill_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, kv_start: torch.Tensor, max_len: int,
                          sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                          causal: bool = True, stream=None) -> None:
    """Causal FP16 prefill over contiguous K/V rows (see ekv.h).

    q: [T, Hq, D]; k, v: [R, Hkv, D] (or the workspace view [pages, 16, Hkv, D])."""
    _expect(q.dim() == 3, f"q must be [rows, num_q_heads, head_dim], got {tuple(q.shape)}")
    q_rows, hq, d = q.shape
    _expect(k.dim() in (3, 4), f"k must be [rows, Hkv, D] or [pages, 16, Hkv, D], got {tuple(k.shape)}")
    _expect(k.dim() == 3 or int(k.shape[1]) == PAGE_SIZE, f"workspace pages hold {PAGE_SIZE} rows, got {tuple(k.shape)}")
    _expect(kv_start.dim() == 1 and tuple(cu_seqlens_q.shape) == (int(kv_start.shape[0]) + 1,),
            f"cu_seqlens_q must have n_prompts + 1 = {int(kv_start.shape[0]) + 1} entries, got "
            f"{tuple(cu_seqlens_q.shape)}")
    _check_prefill_out(q, out, lse)
    hkv = int(k.shape[-2])
    if int(k.shape[-1]) != d:
        raise ValueError(f"K rows have head dim {int(k.shape[-1])}, queries {d}")
    _same_shape(k, v, "k and v")
    kv_rows = k.numel() // (hkv * d)
    _check(_lib.ekv_prefill_attention(
        _arg(q, "q", _F16), q_rows, _arg(k, "k", _F16), _arg(v, "v", _F16), kv_rows,
        _arg(cu_seqlens_q, "cu_seqlens_q", _I32), _arg(kv_start, "kv_start", _I32),
        int(kv_start.shape[0]), int(max_len), hq, hkv, d, 1 if causal else 0, float(sm_scale),
        _arg(out, "out"), _dtype_code(out), _arg(lse, "lse", _F32), _stream(stream)))


def ekv_prefill_paged_attention(kv: PagedKV, q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                page_table: torch.Tensor, fidelity: Optional[torch.Tensor], max_len: int,
                                sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                                causal: bool = True, stream=None) -> None:
    """Causal FP16 prefill straight from each prompt's pages (see ekv.h).

    q: [T, Hq, D]; page_table: [n_prompts, stride] int32; fidelity: same shape uint8 or None."""
    _expect(q.dim() == 3, f"q must be [rows, num_q_heads, head_dim], got {tuple(q.shape)}")
    _expect(int(q.shape[2]) == kv.head_dim, f"q has head dim {int(q.shape[2])}, the pools {kv.head_dim}")
    _expect(page_table.dim() == 2 and tuple(cu_seqlens_q.shape) == (int(page_table.shape[0]) + 1,),
            f"cu_seqlens_q must have one entry per page-table row plus one, got {tuple(cu_seqlens_q.shape)} "
            f"for page_table {tuple(page_table.shape)}")
    _check_prefill_out(q, out, lse)
    q_rows, hq, _ = q.shape
    _same_shape(page_table, fidelity, "page_table and fidelity")
    _check(_lib.ekv_prefill_paged_attention(
        _kv_ref(kv), _arg(q, "q", _F16), q_rows, _arg(cu_seqlens_q, "cu_seqlens_q", _I32),
        _arg(page_table, "page_table", _I32), int(page_table.shape[1]), _arg(fidelity, "fidelity", _U8),
        int(page_table.shape[0]), int(max_len), hq, 1 if causal else 0, float(sm_scale),
        _arg(out, "out"), _dtype_code(out), _arg(lse, "lse", _F32), _stream(stream)))


def ekv_append_tokens(kv: PagedKV, k_new: torch.Tensor, v_new: torch.Tensor,
                      slot_mapping: torch.Tensor, stream=None) -> None:
    """Write new tokens' K/V rows ([n, Hkv, D] fp16) into TARGET slots (see ekv.h).
    ``kv`` must describe writable TARGET pools."""
    _same_shape(k_new, v_new, "k_new and v_new")
    _expect(tuple(k_new.shape[-2:]) == (kv.num_kv_heads, kv.head_dim),
            f"k_new rows must be [{kv.num_kv_heads}, {kv.head_dim}], got {tuple(k_new.shape)}")
    if k_new.numel() != int(slot_mapping.shape[0]) * kv.num_kv_heads * kv.head_dim:
        raise ValueError("k_new/v_new must hold one [Hkv, D] row per slot_mapping entry")
    _check(_lib.ekv_append_tokens(_kv_ref(kv), _arg(k_new, "k_new", _F16), _arg(v_new, "v_new", _F16),
                                  _arg(slot_mapping, "slot_mapping", _I32), int(slot_mapping.shape[0]),
                                  _stream(stream)))


def ekv_quantize_pages(kv: PagedKV, k_src: torch.Tensor, v_src: torch.Tensor,
                       src_row_start: torch.Tensor, dst_pages: torch.Tensor,
                       n_valid: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write compact pages (K16 + E4M3 V + per-page-per-head scale) from fp16 rows (see ekv.h).

    k_src, v_src: [rows, Hkv, D] (or the TARGET pool view [pages, 16, Hkv, D]).
    ``kv`` must describe writable compact pools."""
    _same_shape(k_src, v_src, "k_src and v_src")
    _same_shape(src_row_start, dst_pages, "src_row_start and dst_pages")
    _same_shape(n_valid, dst_pages, "n_valid and dst_pages")
    _expect(tuple(k_src.shape[-2:]) == (kv.num_kv_heads, kv.head_dim),
            f"k_src rows must be [{kv.num_kv_heads}, {kv.head_dim}], got {tuple(k_src.shape)}")
    rows = k_src.numel() // (kv.num_kv_heads * kv.head_dim)
    _check(_lib.ekv_quantize_pages(_kv_ref(kv), _arg(k_src, "k_src", _F16), _arg(v_src, "v_src", _F16),
                                   rows, _arg(src_row_start, "src_row_start", _I32),
                                   _arg(n_valid, "n_valid", _I32), _arg(dst_pages, "dst_pages", _I32),
                                   int(dst_pages.shape[0]), _stream(stream)))


def ekv_e4m3_to_f16(codes: torch.Tensor, out: torch.Tensor, method: int, scale_exp: int = 0,
                    stream=None) -> None:
    """Diagnostic: device E4M3 -> fp16 of code * 2^scale_exp (0 = decode path, 1 = gather path)."""
    if out.numel() != codes.numel():
        raise ValueError("out must hold one fp16 value per code")
    _check(_lib.ekv_e4m3_to_f16(_arg(codes, "codes", _U8), int(codes.numel()), _arg(out, "out", _F16),
                                int(method), int(scale_exp), _stream(stream)))

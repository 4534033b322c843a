"""C-ABI checks that need no GPU: the library loads, exports every function
include/ekv.h declares, and host-side validation returns the documented
status before any launch (all cases below are rejected on the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ekv.h")

ekv = pytest.importorskip("mixed_precision_paged_amd.ekv", reason="libekv.so not built")

FAKE = 0x10000  # aligned non-null address; never dereferenced: every call below fails validation


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(ekv_\w+)\s*\(", text, re.M)))


def test_every_declared_function_is_exported():
    names = _declared()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(ekv._lib, n), n
    assert sorted(ekv.EXPORTED) == names


def test_library_was_built_from_these_sources():
    from mixed_precision_paged_amd import build

    assert len(ekv.ekv_build_id()) == 64
    build.check_library_matches_sources()


def test_version_and_status_strings():
    assert ekv.ekv_abi_version() == 1
    assert ekv.ekv_status_string(ekv.EKV_OK) == "ok"
    assert "workspace" in ekv.ekv_status_string(ekv.EKV_ERR_WORKSPACE_TOO_SMALL)
    assert ekv.ekv_status_string(99) == "unknown status"


def _kv(hkv=8, d=128, page=16, n_t=0, n_c=100):
    return ekv.PagedKV(FAKE if n_t else None, FAKE if n_t else None, n_t,
                       FAKE if n_c else None, FAKE if n_c else None, FAKE if n_c else None, n_c,
                       hkv, d, page)


def _decode(kv, hq=32, batch=4, pt_stride=512, fidelity=FAKE, max_len=8192, scratch=FAKE,
            scratch_bytes=1 << 30, pps=0, out_dtype=0, q=FAKE):
    return ekv._lib.ekv_decode_attention(ctypes.byref(kv) if kv is not None else None, q, batch, hq,
                                         FAKE, pt_stride, fidelity, FAKE, max_len, 0.088, FAKE,
                                         out_dtype, None, pps, scratch, scratch_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(hq=30), ekv.EKV_ERR_INVALID_ARG),          # Hq % Hkv != 0
    (dict(hq=24), ekv.EKV_ERR_UNSUPPORTED),          # G = 3
    (dict(pt_stride=100), ekv.EKV_ERR_INVALID_ARG),  # stride < ceil(max_len / 16)
    (dict(scratch=None), ekv.EKV_ERR_INVALID_ARG),
    (dict(scratch_bytes=16), ekv.EKV_ERR_INVALID_ARG),
    (dict(scratch=FAKE + 16), ekv.EKV_ERR_INVALID_ARG),  # scratch not 256-byte aligned
    (dict(pps=5000), ekv.EKV_ERR_INVALID_ARG),
    (dict(out_dtype=7), ekv.EKV_ERR_INVALID_ARG),
    (dict(q=None), ekv.EKV_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), ekv.EKV_ERR_INVALID_ARG),     # misaligned query
])
def test_decode_validation(kwargs, status):
    assert _decode(_kv(), **kwargs) == status
    assert ekv.ekv_last_error() != ""


def test_decode_validation_of_pools():
    assert _decode(None) == ekv.EKV_ERR_INVALID_ARG
    assert _decode(_kv(d=96)) == ekv.EKV_ERR_UNSUPPORTED
    assert _decode(_kv(page=8)) == ekv.EKV_ERR_INVALID_ARG
    assert _decode(_kv(n_t=5, n_c=5), fidelity=None) == ekv.EKV_ERR_INVALID_ARG
    bad = _kv()
    bad.v_scale = None
    assert _decode(bad) == ekv.EKV_ERR_INVALID_ARG


def test_decode_empty_batch_is_ok_without_launch():
    assert _decode(_kv(), batch=0) == ekv.EKV_OK
    assert ekv.ekv_last_error() == ""


def test_split_plan_and_scratch_size():
    # 256 (sequence, KV head) groups: one split each, no partials
    assert ekv.ekv_decode_pages_per_split(32, 8, 8192) == 512
    assert ekv.ekv_decode_scratch_bytes(32, 32, 8, 128, 8192, 0) == 0
    up = lambda n: (n + 255) // 256 * 256

    def split_scratch(batch, hq, hkv, d, splits):  # acc | (max, sum) per (b, q head, split)
        rows = batch * hq * splits
        return up(rows * d * 4) + rows * 2 * 4

    for pps, splits in ((256, 2), (128, 4), (100, 6)):
        assert ekv.ekv_decode_scratch_bytes(32, 32, 8, 128, 8192, pps) == split_scratch(32, 32, 8, 128, splits)
    # 128 groups: about 512 split workgroups of pages
    assert ekv.ekv_decode_pages_per_split(16, 8, 8192) == 128
    # 512 groups: one split each
    assert ekv.ekv_decode_pages_per_split(64, 8, 8192) == 512
    # balanced plan: 512 workgroups (two rounds of 256) x 2 partial records of G x (D + 2) floats
    bal = ekv.ekv_decode_scratch_bytes(64, 32, 8, 128, 8192, ekv.DECODE_BALANCED)
    recs = 512 * 2 * 4
    assert bal == ((recs * 128 * 4 + 255) // 256) * 256 + recs * 2 * 4
    # whole rounds more once a share could pass 512 pages: 64 x 8 x 2048 pages -> 2048
    recs = 2048 * 2 * 4
    assert ekv.ekv_decode_scratch_bytes(64, 32, 8, 128, 32768, ekv.DECODE_BALANCED) == \
        ((recs * 128 * 4 + 255) // 256) * 256 + recs * 2 * 4
    assert ekv.ekv_decode_scratch_bytes(2, 4, 1, 64, 64, 1) == split_scratch(2, 4, 1, 64, 4)
    assert ekv.ekv_decode_scratch_bytes(0, 4, 1, 64, 64, 1) == 0


def test_split_plan_from_host_lengths():
    import numpy as np
    uniform = ekv.ekv_decode_plan_pages_per_split(np.full(32, 8192), 8)
    assert uniform == ekv.ekv_decode_pages_per_split(32, 8, 8192) == 512
    lens = np.random.default_rng(0).integers(1024, 16385, size=64)
    assert ekv.ekv_decode_plan_pages_per_split(lens, 8) == ekv.DECODE_BALANCED
    # beyond the balanced plan's batch limit: small splits
    big = np.random.default_rng(0).integers(64, 1025, size=2049)
    ragged = ekv.ekv_decode_plan_pages_per_split(big, 8)
    pages = int(((big + 15) // 16).sum())
    assert ragged % 4 == 0 and 16 <= ragged <= 512 and abs(ragged - pages * 8 / 4096) <= 4
    assert ekv.ekv_decode_plan_pages_per_split([], 8) == 16
    assert ekv.ekv_decode_plan_pages_per_split([0, 0], 8) == 16
    # near-equal lengths whose split plan would launch more than one round of 4-wavefront
    # workgroups (n > 768), or at most 32 (sequence, KV head) groups of 2,048+ pages, get
    # equal shares instead; otherwise splits
    for b, ctx in ((128, 8192), (32, 32768), (128, 2048), (64, 32768), (128, 32768), (1, 32768), (4, 32768)):
        assert ekv.ekv_decode_plan_pages_per_split(np.full(b, ctx), 8) == ekv.DECODE_BALANCED, (b, ctx)
    for b, ctx, pps in ((64, 8192, 512), (16, 32768, 512), (16, 8192, 128), (1, 8192, 16), (64, 2048, 128)):
        assert ekv.ekv_decode_plan_pages_per_split(np.full(b, ctx), 8) == pps, (b, ctx)


def test_gather_validation():
    kv = _kv()
    g = ekv._lib.ekv_gather_compact_pages
    assert g(ctypes.byref(kv), FAKE, 4097, 1, FAKE, FAKE, 4096, None) == ekv.EKV_ERR_WORKSPACE_TOO_SMALL
    assert g(ctypes.byref(kv), FAKE, 4, 2, FAKE, FAKE, 4096, None) == ekv.EKV_ERR_INVALID_ARG
    assert g(ctypes.byref(kv), None, 4, 1, FAKE, FAKE, 4096, None) == ekv.EKV_ERR_INVALID_ARG
    assert g(ctypes.byref(_kv(d=32)), FAKE, 4, 1, FAKE, FAKE, 4096, None) == ekv.EKV_ERR_UNSUPPORTED
    no_c = _kv(n_t=4, n_c=0)
    assert g(ctypes.byref(no_c), FAKE, 4, 1, FAKE, FAKE, 4096, None) == ekv.EKV_ERR_INVALID_ARG
    assert g(ctypes.byref(kv), FAKE, 0, 1, FAKE, FAKE, 4096, None) == ekv.EKV_OK


def _prefill(max_len=8192, hq=32, hkv=8, d=128, causal=1, out=FAKE, sm_scale=0.088):
    return ekv._lib.ekv_prefill_attention(FAKE, 1000, FAKE, FAKE, 1000, FAKE, FAKE, 2, max_len, hq,
                                          hkv, d, causal, sm_scale, out, 0, None, None)


def test_prefill_validation():
    assert _prefill(max_len=8193) == ekv.EKV_ERR_NOT_ELIGIBLE
    assert _prefill(hq=33) == ekv.EKV_ERR_INVALID_ARG
    assert _prefill(d=80) == ekv.EKV_ERR_UNSUPPORTED
    assert _prefill(causal=2) == ekv.EKV_ERR_INVALID_ARG
    assert _prefill(out=None) == ekv.EKV_ERR_INVALID_ARG
    for bad in (0.0, -0.088, float("nan"), float("inf")):  # the kernels need a positive scale
        assert _prefill(sm_scale=bad) == ekv.EKV_ERR_INVALID_ARG, bad
    assert _prefill(max_len=0) == ekv.EKV_OK


def test_e4m3_diagnostic_validation():
    f = ekv._lib.ekv_e4m3_to_f16
    assert f(FAKE, 4, FAKE, 2, 0, None) == ekv.EKV_ERR_INVALID_ARG   # method
    assert f(FAKE, 4, FAKE, 0, 128, None) == ekv.EKV_ERR_INVALID_ARG  # exponent beyond fp32 normals
    assert f(FAKE, 4, FAKE, 1, -127, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(None, 4, FAKE, 0, 0, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(FAKE, 0, FAKE, 0, -33, None) == ekv.EKV_OK


def test_append_validation():
    f = ekv._lib.ekv_append_tokens
    kv_t = _kv(n_t=64, n_c=0)
    assert f(ctypes.byref(_kv(n_t=0, n_c=5)), FAKE, FAKE, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv_t), None, FAKE, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv_t), FAKE + 8, FAKE, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv_t), FAKE, FAKE, FAKE, -1, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(_kv(d=96, n_t=64)), FAKE, FAKE, FAKE, 4, None) == ekv.EKV_ERR_UNSUPPORTED
    assert f(ctypes.byref(_kv(n_t=1 << 28, n_c=0)), FAKE, FAKE, FAKE, 4, None) == ekv.EKV_ERR_UNSUPPORTED
    assert f(None, FAKE, FAKE, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv_t), FAKE, FAKE, FAKE, 0, None) == ekv.EKV_OK


def test_quantize_validation():
    f = ekv._lib.ekv_quantize_pages
    kv = _kv()
    assert f(ctypes.byref(_kv(n_t=5, n_c=0)), FAKE, FAKE, 64, FAKE, None, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv), FAKE, FAKE, 64, None, None, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv), FAKE, FAKE, 64, FAKE, None, None, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv), FAKE, FAKE + 4, 64, FAKE, None, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv), FAKE, FAKE, -1, FAKE, None, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(_kv(d=32)), FAKE, FAKE, 64, FAKE, None, FAKE, 4, None) == ekv.EKV_ERR_UNSUPPORTED
    assert f(ctypes.byref(kv), FAKE, FAKE, 64, FAKE, None, FAKE, 0, None) == ekv.EKV_OK


def _paged_prefill(kv, max_len=8192, hq=32, causal=1, out=FAKE, pt_stride=512, fidelity=FAKE, sm_scale=0.088):
    return ekv._lib.ekv_prefill_paged_attention(ctypes.byref(kv) if kv is not None else None, FAKE, 1000,
                                                FAKE, FAKE, pt_stride, fidelity, 2, max_len, hq, causal,
                                                sm_scale, out, 0, None, None)


def test_paged_prefill_validation():
    kv = _kv()
    assert _paged_prefill(kv, max_len=8193, pt_stride=600) == ekv.EKV_ERR_NOT_ELIGIBLE
    assert _paged_prefill(kv, hq=33) == ekv.EKV_ERR_INVALID_ARG
    assert _paged_prefill(_kv(d=80)) == ekv.EKV_ERR_UNSUPPORTED
    assert _paged_prefill(kv, causal=2) == ekv.EKV_ERR_INVALID_ARG
    assert _paged_prefill(kv, out=None) == ekv.EKV_ERR_INVALID_ARG
    assert _paged_prefill(kv, pt_stride=100) == ekv.EKV_ERR_INVALID_ARG
    assert _paged_prefill(_kv(n_t=5, n_c=5), fidelity=None) == ekv.EKV_ERR_INVALID_ARG
    assert _paged_prefill(None) == ekv.EKV_ERR_INVALID_ARG
    for bad in (0.0, -0.088, float("nan")):
        assert _paged_prefill(kv, sm_scale=bad) == ekv.EKV_ERR_INVALID_ARG, bad
    assert _paged_prefill(kv, max_len=0) == ekv.EKV_OK


def _elastic(kv, fidelity=FAKE, bounds=None, has_base=1):
    return ekv._lib.ekv_decode_attention_elastic(ctypes.byref(kv), FAKE, 4, 32, FAKE, 512, fidelity, bounds,
                                                 has_base, FAKE, 8192, 0.088, FAKE, 0, None, 0, FAKE,
                                                 1 << 30, None)


def test_elastic_decode_validation():
    kv = _kv(n_t=64, n_c=0)
    assert _elastic(kv, fidelity=FAKE, bounds=FAKE) == ekv.EKV_ERR_INVALID_ARG      # both given
    assert _elastic(kv, fidelity=None, bounds=None) == ekv.EKV_ERR_INVALID_ARG      # neither given
    assert _elastic(_kv(n_t=0, n_c=8), fidelity=FAKE) == ekv.EKV_ERR_INVALID_ARG   # no TARGET pool
    assert _elastic(kv, fidelity=None, bounds=FAKE, has_base=0) == ekv.EKV_ERR_INVALID_ARG
    assert _elastic(kv, has_base=2) == ekv.EKV_ERR_INVALID_ARG
    assert _elastic(_kv(n_t=1 << 28, n_c=0)) == ekv.EKV_ERR_UNSUPPORTED


def test_pack_validation():
    f = ekv._lib.ekv_pack_base_pairs
    kv = _kv(n_t=64, n_c=0)
    assert f(ctypes.byref(_kv(n_t=0, n_c=5)), FAKE, FAKE, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv), None, FAKE, FAKE, 4, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(kv), FAKE, FAKE, FAKE, -1, None) == ekv.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(_kv(hkv=32, n_t=64, n_c=0)), FAKE, FAKE, FAKE, 4, None) == ekv.EKV_ERR_UNSUPPORTED
    assert f(ctypes.byref(kv), FAKE, FAKE, FAKE, 0, None) == ekv.EKV_OK


def test_descriptor_keeps_its_tensors_alive():
    """paged_kv(...) on temporaries must not leave dangling device pointers."""
    import gc
    import weakref

    import torch

    t = torch.zeros((2, 16, 1, 64), dtype=torch.float16)
    ref = weakref.ref(t)
    kv = ekv.paged_kv(1, 64, t, t.clone())
    del t
    gc.collect()
    assert ref() is not None and kv._tensors[0] is ref()


def test_binding_rejects_host_tensors_and_bad_shapes():
    """The Python binding refuses, before any library call, tensors that would hand the
    kernels host addresses, and shape pairs the entry points assume equal."""
    import torch

    kv = ekv.paged_kv(8, 128, k_compact=torch.zeros((4, 16, 8, 128), dtype=torch.float16),
                      v_compact=torch.zeros((4, 16, 8, 128), dtype=torch.uint8),
                      v_scale=torch.ones((4, 8), dtype=torch.float32))
    q = torch.zeros((1, 32, 128), dtype=torch.float16)
    pt = torch.zeros((1, 4), dtype=torch.int32)
    lens = torch.full((1,), 64, dtype=torch.int32)
    out = torch.zeros((1, 32, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        ekv.ekv_decode_attention(kv, q, pt, None, lens, 64, 0.088, out)
    with pytest.raises(ValueError, match="device"):
        ekv.ekv_prefill_attention(q, torch.zeros((16, 8, 128), dtype=torch.float16),
                                  torch.zeros((16, 8, 128), dtype=torch.float16),
                                  torch.zeros(2, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                                  1, 0.088, out)
    with pytest.raises(ValueError, match="differ"):
        ekv.ekv_prefill_attention(q, torch.zeros((16, 8, 128), dtype=torch.float16),
                                  torch.zeros((8, 8, 128), dtype=torch.float16),
                                  torch.zeros(2, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                                  1, 0.088, out)
    ids = torch.zeros(2, dtype=torch.int32)
    ws = torch.zeros((4, 16, 8, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="exceeds"):
        ekv.ekv_gather_compact_pages(kv, ids, True, ws, ws, n_pages=3)
    with pytest.raises(ValueError, match="differ"):
        ekv.ekv_decode_attention(kv, q, pt, torch.zeros((1, 5), dtype=torch.uint8), lens, 64, 0.088, out)


def test_binding_rejects_shape_mismatches_before_any_call():
    """Shapes the entry points take on trust -- workspace pages, output and LSE sizes, one
    page-table row and one length per sequence, n_prompts + 1 offsets, matching head dims --
    are checked by the binding and raise before the library is called (host tensors here:
    a shape error is raised before the device check)."""
    import torch

    f16, f32, i32, u8 = torch.float16, torch.float32, torch.int32, torch.uint8
    kv = ekv.paged_kv(8, 128, k_compact=torch.zeros((4, 16, 8, 128), dtype=f16),
                      v_compact=torch.zeros((4, 16, 8, 128), dtype=u8), v_scale=torch.ones((4, 8), dtype=f32))
    q = torch.zeros((2, 32, 128), dtype=f16)
    pt = torch.zeros((2, 4), dtype=i32)
    lens = torch.full((2,), 64, dtype=i32)
    out = torch.zeros((2, 32, 128), dtype=f32)
    lse = torch.zeros((2, 32), dtype=f32)
    dec = ekv.ekv_decode_attention
    bad_decode = [
        dict(q=torch.zeros((2, 32, 64), dtype=f16), out=torch.zeros((2, 32, 64), dtype=f32)),  # head dim 64 vs 128
        dict(page_table=torch.zeros((3, 4), dtype=i32)),     # rows != batch
        dict(seq_lens=torch.full((3,), 64, dtype=i32)),     # lengths != batch
        dict(out=torch.zeros((2, 32, 64), dtype=f32)),      # out smaller than q
        dict(lse=torch.zeros((2, 16), dtype=f32)),          # lse of the wrong size
    ]
    for bad in bad_decode:
        a = dict(q=q, page_table=pt, seq_lens=lens, out=out, lse=lse)
        a.update(bad)
        for fn in (dec, ekv.ekv_decode_attention_noalloc):
            with pytest.raises(ValueError):
                fn(kv, a["q"], a["page_table"], None, a["seq_lens"], 64, 0.088, a["out"], a["lse"])
    with pytest.raises(ValueError, match="base_bounds"):
        ekv.ekv_decode_attention_elastic(kv, q, pt, None, torch.zeros((2, 3), dtype=i32), True, lens, 64, 0.088,
                                         out)
    ids = torch.zeros(2, dtype=i32)
    rows = torch.zeros((64, 8, 128), dtype=f16)            # a row view: 16x the pages it would claim
    ws = torch.zeros((4, 16, 8, 128), dtype=f16)
    with pytest.raises(ValueError, match="ws_k must be"):
        ekv.ekv_gather_compact_pages(kv, ids, True, rows, rows)
    with pytest.raises(ValueError, match="ws_v must be"):
        ekv.ekv_gather_compact_pages(kv, ids, True, ws, torch.zeros((4, 16, 8, 64), dtype=f16))
    pq = torch.zeros((32, 32, 128), dtype=f16)
    pout = torch.zeros((32, 32, 128), dtype=f32)
    k = torch.zeros((32, 8, 128), dtype=f16)
    cu = torch.tensor([0, 16, 32], dtype=i32)
    ks = torch.tensor([0, 16], dtype=i32)
    with pytest.raises(ValueError, match="n_prompts"):
        ekv.ekv_prefill_attention(pq, k, k, cu[:2], ks, 16, 0.088, pout)
    with pytest.raises(ValueError, match="out must be"):
        ekv.ekv_prefill_attention(pq, k, k, cu, ks, 16, 0.088, pout[:16])
    with pytest.raises(ValueError, match="lse must be"):
        ekv.ekv_prefill_attention(pq, k, k, cu, ks, 16, 0.088, pout, torch.zeros((32, 8), dtype=f32))
    with pytest.raises(ValueError, match="head dim"):
        ekv.ekv_prefill_attention(pq, torch.zeros((32, 8, 64), dtype=f16), torch.zeros((32, 8, 64), dtype=f16),
                                  cu, ks, 16, 0.088, pout)
    with pytest.raises(ValueError, match="cu_seqlens_q"):
        ekv.ekv_prefill_paged_attention(kv, pq, cu, torch.zeros((3, 2), dtype=i32), None, 16, 0.088, pout)
    with pytest.raises(ValueError, match="head dim"):
        ekv.ekv_prefill_paged_attention(kv, torch.zeros((32, 32, 64), dtype=f16), cu,
                                        torch.zeros((2, 2), dtype=i32), None, 16, 0.088,
                                        torch.zeros((32, 32, 64), dtype=f32))
    with pytest.raises(ValueError, match="out must be"):
        ekv.ekv_prefill_paged_attention(kv, pq, cu, torch.zeros((2, 2), dtype=i32), None, 16, 0.088, pout[:8])


@pytest.mark.parametrize("workload", ["decode", "prefill", "mixed", "writer", "elastic"])
def test_bench_refuses_more_than_one_gpu(workload):
    """bench.py runs on one GPU only; asking for more exits with status 2 and says why,
    before touching any device."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--workload", workload],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_noalloc_decode_rejects_plans_beyond_its_static_scratch():
    """The allocation-free decode refuses, on the host and before any device call, a plan
    whose partial results would not fit its 8 MiB static scratch."""
    need = ekv.ekv_decode_scratch_bytes(2048, 32, 8, 128, 65536, 1)
    assert need > ekv.NOALLOC_SCRATCH_BYTES
    st = ekv._lib.ekv_decode_attention_noalloc(ctypes.byref(_kv()), FAKE, 2048, 32, FAKE, 4096, FAKE, FAKE,
                                               65536, 0.088, FAKE, 0, None, 1, None)
    assert st == ekv.EKV_ERR_WORKSPACE_TOO_SMALL
    assert "static decode scratch" in ekv.ekv_last_error()


def test_bench_cpu_baseline_pool_runs_the_oracle():
    """bench.py's CPU baseline: a spawned pool runs the unchanged oracle over (sequence, KV
    head) tasks on inputs shared through a memory-mapped file, and reports its worker count."""
    import sys

    sys.path.insert(0, ROOT)
    import bench
    from mixed_precision_paged_amd import bytemodel, synth

    c = synth.make_paged_case(5, [40, 100], 8, 2, 64, compact_frac=0.5)
    ab = bytemodel.decode_bytes(c.seq_lens, c.fidelity, 8, 2, 64)
    r = bench.cpu_decode_baseline(c, ab, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert 1 <= r["cores"] <= bench.CPU_WORKERS_MAX
    assert "4 (sequence, KV head) tasks" in r["sample"]


def test_bench_counted_traffic_follows_the_kernel_source(monkeypatch):
    """bench.py reports a kernel's counted HBM traffic only while the committed counter
    record's source hash matches the kernel's sources (comments and spacing aside)."""
    import sys

    sys.path.insert(0, ROOT)
    import bench

    rec = bench.pmc_record("prefill_route_32x8192_pmc.md")
    assert rec["traffic_bytes_per_call"] >= rec["algorithmic_bytes_per_call"] > 0
    h = bench.prefill_code_hash()
    monkeypatch.setattr(bench, "prefill_code_hash", lambda: h)
    want = int(rec["traffic_bytes_per_call"]) if rec["kernel_code_sha256"] == h else None
    assert bench.counted_prefill_traffic() == want
    monkeypatch.setattr(bench, "prefill_code_hash", lambda: "0" * 64)
    assert bench.counted_prefill_traffic() is None
    # a comment or a change of spacing leaves the hash alone; code does not
    src = os.path.join(ROOT, "mixed_precision_paged_amd", "csrc", "prefill.hip")
    text = open(src).read()
    real_open = open

    def fake_open(path, *a, **k):
        if os.path.abspath(str(path)) == os.path.abspath(src):
            import io
            return io.StringIO(fake_open.text)
        return real_open(path, *a, **k)

    monkeypatch.setattr("builtins.open", fake_open)
    fake_open.text = "// a new comment\n" + text.replace("\n", "\n  ", 3)
    with_comment = bench.code_hash(("prefill.hip",))
    fake_open.text = text
    plain = bench.code_hash(("prefill.hip",))
    assert with_comment == plain
    fake_open.text = text + "\nint extra_symbol;\n"
    assert bench.code_hash(("prefill.hip",)) != plain

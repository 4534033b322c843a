"""Compact-page gather into the FP16 prefill workspace.

[asym] "What changes in vLLM's prefill routing?" (figure "Fresh prefill gets
a fast path inside a mixed batch"): stored K16/V8 pages are gathered into one
bounded FP16 workspace (at most 4,096 pages) and the FP8 values are cast to
FP16; casting does not recover lost precision.

Readings taken where the pages leave it open: workspace page i holds the
page ``page_ids[i]`` in the pool's own [16, Hkv, D] layout, so the workspace
is token-major [n * 16, Hkv, D].  Keys are copied bit for bit.  Values:
  unscaled:  fp16(e4m3(byte))                     (exact: every finite E4M3
                                                   value is an FP16 value)
  scaled:    fp16(fp32(e4m3(byte)) * fp32(scale))  (one fp32 multiply rounded
                                                   to nearest even, then one
                                                   fp16 rounding to nearest
                                                   even)
E4M3 NaN codes become FP16 NaN (payload unspecified).
"""
import numpy as np

from .e4m3 import decode_e4m3fn


def gather_compact_pages(k_compact, v_compact, v_scale, page_ids, apply_scale):
    """Returns (ws_k, ws_v), both float16 [n, 16, Hkv, D]."""
    ids = np.asarray(page_ids, dtype=np.int64)
    ws_k = np.asarray(k_compact)[ids].copy()
    vals = decode_e4m3fn(np.asarray(v_compact)[ids])            # float64, exact
    if apply_scale:
        s32 = np.asarray(v_scale, dtype=np.float32)[ids]        # [n, Hkv]
        prod = vals.astype(np.float32) * s32[:, None, :, None]  # float32 multiply
        ws_v = prod.astype(np.float16)
    else:
        ws_v = vals.astype(np.float16)
    return ws_k, ws_v

"""Cache writer: token append into TARGET pages and TARGET -> compact page conversion.

Test infrastructure only (the oracle): tests, the smoke check and the bench's
CPU baseline may call it; the product path never does.

[ekv] section 3.2 and appendix B.3: newly appended KV is stored at target
fidelity in the protected recent window; section 3.3 and appendix B.2: a
TARGET -> compact transition (demotion) rewrites whole pages.  [asym] "What
changes in vLLM's prefill routing?" and the table "Historical reported
implementation checks": the compact page keeps K bit for bit and holds V as
E4M3 codes with value scales, the writer's V error being FP8 rounding only.

Readings taken where the pages leave it open:
  * append: token i goes to TARGET page slot_page[i], slot slot_index[i]; its
    K and V rows (all KV heads) are copied bit for bit;
  * compaction of a page with n valid tokens (1..16), per KV head h:
      scale[h] = fp32(absmax of the fp16 V over the n valid tokens x D) / 448
                 (one fp32 division, round to nearest even); 1.0 if absmax is 0
      code     = E4M3FN(fp32(v) / scale[h]) for every slot of the page
                 (fp32 division, then round to nearest even on the E4M3 grid;
                 magnitudes at or above 448 saturate to 448; NaN -> 0x7F)
      K        = bit copy of every slot.
    Valid rows must hold finite values; rows past n are encoded too, but
    their contents do not enter the scale.
"""
import math

import numpy as np

E4M3_MAX = 448.0


def encode_e4m3fn(x: float) -> int:
    """E4M3FN code of x: nearest value, ties to even mantissa, saturating at 448.

    Magnitudes are compared on the value grid: subnormal step 2^-9 below 2^-6,
    then 8 mantissa steps per binade up to 448."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < 2.0 ** -6:                      # subnormal range: multiples of 2^-9
        q = a / 2.0 ** -9                  # exact in float64
        m = _round_half_even(q)
        return sign | m                    # m == 8 is the smallest normal (code 0x08)
    e = math.floor(math.log2(a))
    while 2.0 ** e > a:                    # guard log2 rounding
        e -= 1
    while 2.0 ** (e + 1) <= a:
        e += 1
    q = a / 2.0 ** (e - 3)                 # in [8, 16), exact
    m = _round_half_even(q)                # 8..16
    if m == 16:                            # rounds up into the next binade
        e += 1
        m = 8
    code = ((e + 7) << 3) | (m - 8)
    return sign | min(code, 0x7E)


def _round_half_even(q: float) -> int:
    f = math.floor(q)
    r = q - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        return int(f) + 1
    return int(f)


def encode_e4m3fn_array(x: np.ndarray) -> np.ndarray:
    """encode_e4m3fn over an array, the same steps written with numpy (frexp
    splits a = f * 2^e with f in [0.5, 1), so a / 2^(e-4) = 16 f in [8, 16))."""
    x = np.asarray(x, dtype=np.float64)
    a = np.where(np.isfinite(x), np.abs(x), E4M3_MAX)   # NaN/inf handled below
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.int64)
    f, e = np.frexp(a)
    q = np.rint(16.0 * f)                               # ties to even, 8..16
    e = np.where(q == 16.0, e + 1, e)
    q = np.where(q == 16.0, 8.0, q)
    normal = ((e - 1 + 7) << 3) | (q.astype(np.int64) - 8)
    sub = np.rint(np.minimum(a, 1.0) * 512.0).astype(np.int64)  # subnormal grid 2^-9, 0..8
    code = np.where(a < 2.0 ** -6, sub, normal)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = sign | code
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def compact_page(k16: np.ndarray, v16: np.ndarray, n_valid: int):
    """One TARGET page (fp16 [16, Hkv, D] K and V) -> (K copy, E4M3 codes, fp32 scales [Hkv])."""
    v32 = np.asarray(v16).astype(np.float32)
    hkv = v32.shape[1]
    scale = np.empty(hkv, dtype=np.float32)
    codes = np.empty(v32.shape, dtype=np.uint8)
    for h in range(hkv):
        absmax = np.float32(np.abs(v32[:n_valid, h, :]).max()) if n_valid > 0 else np.float32(0)
        s = np.float32(absmax / np.float32(E4M3_MAX)) if absmax > 0 else np.float32(1.0)
        scale[h] = s
        q = (v32[:, h, :] / s).astype(np.float32)          # fp32 division, RNE
        codes[:, h, :] = encode_e4m3fn_array(q)
    return np.asarray(k16).copy(), codes, scale


def compact_pages(k_target, v_target, src_pages, n_valid):
    """Compaction of the listed TARGET pages: returns (K, codes, scales) per page, stacked."""
    ks, cs, ss = [], [], []
    for p, n in zip(src_pages, n_valid):
        k, c, s = compact_page(k_target[int(p)], v_target[int(p)], int(n))
        ks.append(k)
        cs.append(c)
        ss.append(s)
    return np.stack(ks), np.stack(cs), np.stack(ss)


def append_tokens(k_pool, v_pool, k_new, v_new, slot_page, slot_index):
    """Copies of the pools with token i's K/V rows written at (slot_page[i], slot_index[i])."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for i in range(len(slot_page)):
        k[int(slot_page[i]), int(slot_index[i])] = k_new[i]
        v[int(slot_page[i]), int(slot_index[i])] = v_new[i]
    return k, v

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
  * a compact page is written from n consecutive source token rows
    (0 <= n <= 16; the source is either the TARGET pool seen as rows, for a
    demotion, or freshly computed K/V rows, for a prompt); per KV head h:
      scale[h] = fp32(absmax of the fp16 V over the n rows x D) / 448
                 (one fp32 division, round to nearest even); 1.0 if absmax is 0
      code     = E4M3FN(fp32(v) / scale[h]) for slots 0..n-1
                 (fp32 division, then round to nearest even on the E4M3 grid;
                 magnitudes at or above 448 saturate to 448; NaN -> 0x7F)
      K        = bit copy of slots 0..n-1.
    Slots n..15 are not read from the source (it may end there) and are
    written as zeros (K +0.0, code 0x00).  Source rows must be finite.
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


def quantize_page(k_rows: np.ndarray, v_rows: np.ndarray):
    """n source rows (fp16 [n, Hkv, D] K and V, n <= 16) -> one compact page:
    (K fp16 [16, Hkv, D], E4M3 codes u8 [16, Hkv, D], fp32 scales [Hkv])."""
    k_rows = np.asarray(k_rows, dtype=np.float16)
    v32 = np.asarray(v_rows, dtype=np.float16).astype(np.float32)
    n, hkv, d = v32.shape
    assert n <= 16
    k = np.zeros((16, hkv, d), np.float16)
    k[:n] = k_rows
    codes = np.zeros((16, hkv, d), np.uint8)
    scale = np.empty(hkv, dtype=np.float32)
    for h in range(hkv):
        absmax = np.float32(np.abs(v32[:, h, :]).max()) if n > 0 else np.float32(0)
        s = np.float32(absmax / np.float32(E4M3_MAX)) if absmax > 0 else np.float32(1.0)
        scale[h] = s
        q = (v32[:, h, :] / s).astype(np.float32)          # fp32 division, RNE
        codes[:n, h, :] = encode_e4m3fn_array(q)
    return k, codes, scale


def quantize_pages(k_src, v_src, row_start, n_valid):
    """Page i is written from rows row_start[i] .. row_start[i] + n_valid[i] - 1 of the
    fp16 [rows, Hkv, D] source arrays; returns the stacked (K, codes, scales)."""
    ks, cs, ss = [], [], []
    for r, n in zip(row_start, n_valid):
        r, n = int(r), int(n)
        k, c, s = quantize_page(k_src[r:r + n], v_src[r:r + n])
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

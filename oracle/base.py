"""ElasticKV BASE pages: the high byte of each FP16 value, two pages per block.

[ekv] section 3 (overview): BASE keeps the high-order 8 bits of the 16-bit
TARGET value; the low-order 8 bits refine it back exactly; there are no
quantization parameters.  Section 3.1 and figure 3(b): the two BASE pages of a
logical pair are packed into one TARGET-sized physical block and the other
block is freed.  Section 3.2 and appendix B.3: a BASE value is read by placing
the stored byte in the high-order position and zero-filling the low-order
byte, then reading the 16 bits as the native type.  Appendix B.2: demotion
packs the high-order bytes of the pair's two TARGET blocks on the GPU.

Readings taken where the pages leave it open:
  * BASE page index b lives in TARGET block b // 2: its bytes are half b % 2
    of that block (the first or the second 16 x Hkv x D bytes), laid out
    [slot][kv head][d] like a page;
  * packing pair (a, b) into block dst writes half 0 = high bytes of block a
    and half 1 = high bytes of block b, so the pair's BASE pages are 2 dst
    and 2 dst + 1; K and V pools are packed alike;
  * the fidelity flag of a BASE page is 2.
"""
import numpy as np

BASE = 2


def high_bytes(x16: np.ndarray) -> np.ndarray:
    """High byte of each FP16 value (sign, 5 exponent bits, top 2 mantissa bits)."""
    return (np.asarray(x16, dtype=np.float16).view(np.uint16) >> 8).astype(np.uint8)


def base_values(b8: np.ndarray) -> np.ndarray:
    """FP16 values (as float64) whose high byte is the stored byte and low byte zero."""
    bits = np.asarray(b8, dtype=np.uint16) << 8
    return bits.astype(np.uint16).view(np.float16).astype(np.float64)


def base_page(pool16: np.ndarray, b: int) -> np.ndarray:
    """Bytes [16, Hkv, D] of BASE page b of a TARGET pool fp16 [P, 16, Hkv, D]."""
    P, S, H, D = pool16.shape
    blocks = np.ascontiguousarray(pool16).view(np.uint8).reshape(P, 2, S, H, D)
    return blocks[int(b) // 2, int(b) % 2]


def pack_base_pairs(k_pool16, v_pool16, src_a, src_b, dst):
    """Copies of the pools in which block dst[i] holds the BASE pair of blocks
    (src_a[i], src_b[i]).  Source blocks are read before any block is written."""
    out = []
    for pool in (k_pool16, v_pool16):
        pool = np.asarray(pool, dtype=np.float16)
        P, S, H, D = pool.shape
        hi = {int(x): high_bytes(pool[int(x)]) for x in list(src_a) + list(src_b)}
        new = pool.copy()
        view = new.view(np.uint8).reshape(P, 2, S, H, D)
        for a, b, d in zip(src_a, src_b, dst):
            view[int(d), 0] = hi[int(a)]
            view[int(d), 1] = hi[int(b)]
        out.append(new)
    return out[0], out[1]

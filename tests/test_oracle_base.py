"""Pins for the oracle's ElasticKV BASE pages (high FP16 byte, pair-packed blocks).

A BASE byte is the top 8 bits of FP16: sign, 5 exponent bits, 2 mantissa
bits, i.e. the bit layout of FP8 E5M2.  The library cast torch.float8_e5m2 ->
float64 therefore pins the value of every byte, and brute force over the 256
E5M2 values pins "high byte with zeroed low byte" as truncation toward zero
for every finite FP16 value.  Decode over BASE pages is pinned to float64
SDPA on contiguous tensors built by a test-local packing.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle.base import base_page, base_values, high_bytes, pack_base_pairs

PAGE = 16


def _e5m2_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float64).numpy()


def test_every_byte_matches_library_e5m2():
    lib = _e5m2_values()
    mine = base_values(np.arange(256))
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(lib))
    fin = ~np.isnan(lib)
    np.testing.assert_array_equal(mine[fin], lib[fin])
    assert np.array_equal(np.signbit(mine[fin]), np.signbit(lib[fin]))


def test_base_value_truncates_every_finite_fp16_toward_zero():
    x = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    x = x[np.isfinite(x)]
    got = base_values(high_bytes(x))
    grid = _e5m2_values()
    pos = np.sort(grid[np.isfinite(grid) & (grid >= 0)])
    mag = np.abs(x.astype(np.float64))
    idx = np.searchsorted(pos, mag, side="right") - 1        # largest grid value <= |x|
    want = np.copysign(pos[idx], x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    normal = mag >= 2.0 ** -14
    assert np.all(np.abs(x.astype(np.float64) - got)[normal] < mag[normal] * 2.0 ** -2)


def test_pack_places_high_bytes_in_block_halves_and_allows_in_place():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((6, PAGE, 2, 8)).astype(np.float16)
    v = rng.standard_normal((6, PAGE, 2, 8)).astype(np.float16)
    src_a, src_b, dst = [0, 3], [4, 5], [0, 2]          # pair (0, 4) packed in place into block 0
    k2, v2 = pack_base_pairs(k, v, src_a, src_b, dst)
    for pool, orig in ((k2, k), (v2, v)):
        for a, b, d in zip(src_a, src_b, dst):
            assert np.array_equal(base_page(pool, 2 * d), orig[a].view(np.uint16) >> 8)
            assert np.array_equal(base_page(pool, 2 * d + 1), orig[b].view(np.uint16) >> 8)
        for blk in (1, 3, 4, 5):
            assert np.array_equal(pool[blk].view(np.uint16), orig[blk].view(np.uint16))


def _scatter(rng, keys, vals, modes, extra_blocks=2):
    """Test-local pools: TARGET pages in their own blocks, BASE pages packed two per block
    (independent of the oracle's pack routine).  modes[b][j] in {0 TARGET, 2 BASE}."""
    H, D = keys[0].shape[1], keys[0].shape[2]
    n_t = sum(m.count(0) for m in modes)
    n_b = sum(m.count(2) for m in modes)
    P = n_t + (n_b + 1) // 2 + extra_blocks
    kp = np.full((P, PAGE, H, D), np.nan, np.float16)
    vp = np.full((P, PAGE, H, D), np.nan, np.float16)
    free = list(rng.permutation(P))
    base_slots = []
    table = np.zeros((len(keys), max(len(m) for m in modes)), np.int32)
    flags = np.zeros_like(table, dtype=np.uint8)
    for b, m in enumerate(modes):
        for j, mode in enumerate(m):
            lo, hi = j * PAGE, min(keys[b].shape[0], (j + 1) * PAGE)
            if mode == 0:
                blk = int(free.pop())
                kp[blk, :hi - lo] = keys[b][lo:hi]
                vp[blk, :hi - lo] = vals[b][lo:hi]
                table[b, j] = blk
            else:
                if not base_slots:
                    blk = int(free.pop())
                    base_slots = [2 * blk + 1, 2 * blk]
                    kp[blk] = 0
                    vp[blk] = 0
                bid = base_slots.pop()
                blk, half = bid // 2, bid % 2
                kb = kp[blk].view(np.uint8).reshape(2, PAGE, H, D)
                vb = vp[blk].view(np.uint8).reshape(2, PAGE, H, D)
                kb[half, :hi - lo] = keys[b][lo:hi].view(np.uint16) >> 8
                vb[half, :hi - lo] = vals[b][lo:hi].view(np.uint16) >> 8
                table[b, j] = bid
            flags[b, j] = mode
    return kp, vp, table, flags


def test_decode_with_base_pages_matches_sdpa_on_truncated_values():
    rng = np.random.default_rng(2)
    lens, hq, hkv, d = [70, 33, 16], 8, 2, 32
    keys = [rng.standard_normal((n, hkv, d)).astype(np.float16) for n in lens]
    vals = [rng.standard_normal((n, hkv, d)).astype(np.float16) for n in lens]
    modes = [[0, 2, 2, 0, 2], [2, 0, 2], [2]]
    kp, vp, table, flags = _scatter(rng, keys, vals, modes)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float16)
    sm = 1 / math.sqrt(d)
    empty16 = np.zeros((0, PAGE, hkv, d), np.float16)
    out, lse = oracle.decode_attention(q, kp, vp, empty16, np.zeros((0, PAGE, hkv, d), np.uint8),
                                       np.zeros((0, hkv), np.float32), table, flags,
                                       np.array(lens, np.int32), sm)
    e5m2 = lambda a: torch.from_numpy((a.view(np.uint16) >> 8).astype(np.uint8)).view(
        torch.float8_e5m2).to(torch.float64)
    for b, n in enumerate(lens):
        K = torch.from_numpy(keys[b].astype(np.float64))
        V = torch.from_numpy(vals[b].astype(np.float64))
        for j, mode in enumerate(modes[b]):
            if mode == 2:
                K[j * PAGE:(j + 1) * PAGE] = e5m2(keys[b][j * PAGE:(j + 1) * PAGE])
                V[j * PAGE:(j + 1) * PAGE] = e5m2(vals[b][j * PAGE:(j + 1) * PAGE])
        Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]          # [Hq, 1, D]
        ref = F.scaled_dot_product_attention(Q[None], K.permute(1, 0, 2)[None], V.permute(1, 0, 2)[None],
                                             scale=sm, enable_gqa=True)
        np.testing.assert_allclose(out[b], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_base_page_of_exact_values_equals_target_page():
    """Values whose low byte is already zero lose nothing: BASE == TARGET exactly."""
    rng = np.random.default_rng(3)
    n, hq, hkv, d = 40, 4, 1, 16
    keys = [(rng.standard_normal((n, hkv, d)).astype(np.float16).view(np.uint16) & 0xFF00).view(np.float16)]
    vals = [(rng.standard_normal((n, hkv, d)).astype(np.float16).view(np.uint16) & 0xFF00).view(np.float16)]
    q = rng.standard_normal((1, hq, d)).astype(np.float16)
    kt, vt, tt, ft = _scatter(rng, keys, vals, [[0, 0, 0]])
    kb, vb, tb, fb = _scatter(rng, keys, vals, [[2, 2, 0]])
    z16 = np.zeros((0, PAGE, hkv, d), np.float16)
    z8 = np.zeros((0, PAGE, hkv, d), np.uint8)
    zs = np.zeros((0, hkv), np.float32)
    o1, l1 = oracle.decode_attention(q, kt, vt, z16, z8, zs, tt, ft, np.array([n], np.int32), 0.25)
    o2, l2 = oracle.decode_attention(q, kb, vb, z16, z8, zs, tb, fb, np.array([n], np.int32), 0.25)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)

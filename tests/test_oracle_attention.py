"""Pins for the oracle's paged decode and causal prefill attention.

Pins that do not restate the oracle: torch scaled_dot_product_attention in
float64 on contiguous tensors (library), a scalar brute force on tiny inputs,
closed forms (len 1, q = 0, one-hot keys) and invariants (page permutation,
GQA mapping, compact-with-exact-values == TARGET, prefill row == decode).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_builder import build_paged

PAGE = 16


def _fp8(x32):
    return torch.from_numpy(np.clip(x32, -448, 448).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _random_batch(seed, lens, hq, hkv, d, compact_prob=0.5):
    """Contiguous per-sequence data, then paged via the test-local scatter."""
    rng = np.random.default_rng(seed)
    keys, vals16, codes, scales, flags = [], [], [], [], []
    for n in lens:
        pages = (n + PAGE - 1) // PAGE
        keys.append(rng.standard_normal((n, hkv, d)).astype(np.float16))
        vals16.append(rng.standard_normal((n, hkv, d)).astype(np.float16))
        sc = (rng.uniform(0.5, 2.0, size=(pages, hkv)) / 64).astype(np.float32)
        scales.append(sc)
        codes.append(_fp8(rng.standard_normal((n, hkv, d)) * 40))
        flags.append([int(rng.random() < compact_prob) for _ in range(pages)])
    pools = build_paged(rng, keys, vals16, codes, scales, flags)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float16)
    return q, keys, vals16, codes, scales, flags, pools


def _contiguous_values(vals16, codes, scales, flags):
    """Per-token values in float64 via the LIBRARY float8 cast (not the oracle table)."""
    n = vals16.shape[0]
    out = np.empty(vals16.shape, dtype=np.float64)
    for t in range(n):
        j = t // PAGE
        if flags[j] == 0:
            out[t] = vals16[t].astype(np.float64)
        else:
            lib = torch.from_numpy(codes[t]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            out[t] = lib * scales[j].astype(np.float64)[:, None]
    return out


def _decode(q, pools, sm_scale):
    return oracle.decode_attention(q, pools["k_target"], pools["v_target"], pools["k_compact"],
                                   pools["v_compact"], pools["v_scale"], pools["page_table"],
                                   pools["fidelity"], pools["seq_lens"], sm_scale)


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (8, 2, 32), (6, 3, 16)])
def test_decode_matches_sdpa_float64(hq, hkv, d):
    lens = [1, 15, 16, 17, 37, 64]
    q, keys, vals16, codes, scales, flags, pools = _random_batch(11 + hq, lens, hq, hkv, d)
    sm = 1.0 / math.sqrt(d)
    out, lse = _decode(q, pools, sm)
    for b, n in enumerate(lens):
        K = torch.from_numpy(keys[b].astype(np.float64)).permute(1, 0, 2)[None]      # [1,Hkv,n,D]
        V = torch.from_numpy(_contiguous_values(vals16[b], codes[b], scales[b], flags[b])).permute(1, 0, 2)[None]
        Q = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]               # [1,Hq,1,D]
        ref = F.scaled_dot_product_attention(Q, K, V, scale=sm, enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)
        # log-normalizer against the library logsumexp of the same scores
        Kr = K.repeat_interleave(hq // hkv, dim=1)
        s = (Q @ Kr.transpose(-1, -2))[0, :, 0, :] * sm
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_decode_scalar_brute_force_tiny():
    lens = [3, 18]
    q, keys, vals16, codes, scales, flags, pools = _random_batch(5, lens, 2, 1, 4)
    sm = 0.5
    out, lse = _decode(q, pools, sm)
    for b, n in enumerate(lens):
        V = _contiguous_values(vals16[b], codes[b], scales[b], flags[b])
        for h in range(2):
            sc = [sm * sum(float(q[b, h, i]) * float(keys[b][t, 0, i]) for i in range(4)) for t in range(n)]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            z = sum(w)
            for i in range(4):
                o = sum(w[t] * V[t, 0, i] for t in range(n)) / z
                assert abs(out[b, h, i] - o) < 1e-12
            assert abs(lse[b, h] - (mx + math.log(z))) < 1e-12


def test_decode_page_permutation_invariant():
    lens = [40, 33]
    q, keys, vals16, codes, scales, flags, pools = _random_batch(7, lens, 4, 2, 8)
    out1, lse1 = _decode(q, pools, 0.3)
    rng = np.random.default_rng(99)
    pools2 = build_paged(rng, keys, vals16, codes, scales, flags, extra_pages=9)
    assert not np.array_equal(pools2["page_table"], pools["page_table"])
    out2, lse2 = _decode(q, pools2, 0.3)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_decode_len_one_returns_v0_and_len_zero_is_empty():
    q, keys, vals16, codes, scales, flags, pools = _random_batch(3, [1, 1], 4, 2, 8, compact_prob=0.5)
    out, lse = _decode(q, pools, 0.2)
    for b in range(2):
        V = _contiguous_values(vals16[b], codes[b], scales[b], flags[b])
        for h in range(4):
            np.testing.assert_array_equal(out[b, h], V[0, h // 2])
    pools["seq_lens"] = np.array([0, 1], np.int32)
    out, lse = _decode(q, pools, 0.2)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_decode_zero_query_gives_mean_of_values():
    q, keys, vals16, codes, scales, flags, pools = _random_batch(4, [29], 4, 2, 8)
    q[:] = 0
    out, _ = _decode(q, pools, 1.0)
    V = _contiguous_values(vals16[0], codes[0], scales[0], flags[0])
    for h in range(4):
        np.testing.assert_allclose(out[0, h], V[:, h // 2].mean(axis=0), rtol=0, atol=1e-12)


def test_decode_one_hot_keys_select_one_value():
    d, n = 16, 16
    rng = np.random.default_rng(8)
    alpha = 16.0  # alpha^2 * sm = 64 -> other weights e^-64
    keys = [np.zeros((n, 1, d), np.float16)]
    for t in range(n):
        keys[0][t, 0, t] = alpha
    vals16 = [rng.standard_normal((n, 1, d)).astype(np.float16)]
    codes = [np.zeros((n, 1, d), np.uint8)]
    scales = [np.ones((1, 1), np.float32)]
    pools = build_paged(rng, keys, vals16, codes, scales, [[0]])
    for j in (0, 5, 15):
        q = np.zeros((1, 1, d), np.float16)
        q[0, 0, j] = alpha
        out, _ = _decode(q, pools, 1.0 / 4.0)
        np.testing.assert_allclose(out[0, 0], vals16[0][j, 0].astype(np.float64), rtol=0, atol=1e-15)


def test_decode_gqa_head_mapping():
    """KV head g carries constant value g: query head h must read g = h // (Hq/Hkv)."""
    hq, hkv, d, n = 8, 4, 4, 20
    rng = np.random.default_rng(2)
    keys = [rng.standard_normal((n, hkv, d)).astype(np.float16)]
    vals16 = [np.broadcast_to(np.arange(hkv, dtype=np.float16)[None, :, None], (n, hkv, d)).copy()]
    codes = [np.zeros((n, hkv, d), np.uint8)]
    scales = [np.ones((2, hkv), np.float32)]
    pools = build_paged(rng, keys, vals16, codes, scales, [[0, 0]])
    q = rng.standard_normal((1, hq, d)).astype(np.float16)
    out, _ = _decode(q, pools, 0.5)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], h // 2, rtol=0, atol=1e-12)


def test_identical_queries_in_a_group_give_identical_rows():
    q, keys, vals16, codes, scales, flags, pools = _random_batch(9, [50], 8, 2, 8)
    q[0, 1] = q[0, 0]
    out, lse = _decode(q, pools, 0.3)
    np.testing.assert_array_equal(out[0, 1], out[0, 0])
    assert lse[0, 1] == lse[0, 0]


def test_compact_page_with_exact_values_equals_target_page():
    rng = np.random.default_rng(12)
    n, hkv, d = 32, 2, 8
    keys = [rng.standard_normal((n, hkv, d)).astype(np.float16)]
    codes = [rng.integers(0, 0x7F, size=(n, hkv, d)).astype(np.uint8)]
    codes[0] |= (rng.integers(0, 2, size=codes[0].shape) << 7).astype(np.uint8)
    exact16 = torch.from_numpy(codes[0]).view(torch.float8_e4m3fn).to(torch.float16).numpy()
    scales = [np.ones((2, hkv), np.float32)]
    q = rng.standard_normal((1, 4, d)).astype(np.float16)
    pa = build_paged(np.random.default_rng(1), keys, [exact16], codes, scales, [[1, 1]])
    pb = build_paged(np.random.default_rng(1), keys, [exact16], codes, scales, [[0, 0]])
    pm = build_paged(np.random.default_rng(1), keys, [exact16], codes, scales, [[0, 1]])
    oa, la = _decode(q, pa, 0.4)
    ob, lb = _decode(q, pb, 0.4)
    om, lm = _decode(q, pm, 0.4)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(oa, om)
    np.testing.assert_array_equal(la, lb)


def test_invalid_fidelity_flag_rejected():
    q, keys, vals16, codes, scales, flags, pools = _random_batch(1, [5], 2, 1, 4)
    pools["fidelity"][0, 0] = 3   # 0, 1, 2 are TARGET, COMPACT, BASE
    with pytest.raises(ValueError):
        _decode(q, pools, 0.5)


# ------------------------------------------------------------------ prefill

def _prefill_inputs(seed, lens, hq, hkv, d, gap=16):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    starts, row = [], 0
    for n in lens:
        starts.append(row)
        row += n + gap  # leave unused rows between prompts
    R = row
    k = np.full((R, hkv, d), np.nan, np.float16)
    v = np.full((R, hkv, d), np.nan, np.float16)
    for p, n in enumerate(lens):
        k[starts[p]:starts[p] + n] = rng.standard_normal((n, hkv, d))
        v[starts[p]:starts[p] + n] = rng.standard_normal((n, hkv, d))
    q = rng.standard_normal((int(cu[-1]), hq, d)).astype(np.float16)
    return q, k, v, cu, np.array(starts, np.int32)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (8, 2, 16)])
def test_prefill_matches_sdpa_float64(causal, hq, hkv, d):
    lens = [1, 17, 40, 3]
    q, k, v, cu, starts = _prefill_inputs(21, lens, hq, hkv, d)
    sm = 1.0 / math.sqrt(d)
    out, lse = oracle.prefill_attention(q, k, v, cu, starts, causal, sm)
    for p, n in enumerate(lens):
        Q = torch.from_numpy(q[cu[p]:cu[p + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        K = torch.from_numpy(k[starts[p]:starts[p] + n].astype(np.float64)).permute(1, 0, 2)[None]
        V = torch.from_numpy(v[starts[p]:starts[p] + n].astype(np.float64)).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=sm, enable_gqa=True)
        np.testing.assert_allclose(out[cu[p]:cu[p + 1]], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_prefill_row_subset_matches_full():
    q, k, v, cu, starts = _prefill_inputs(22, [30, 9], 4, 2, 8)
    full, lf = oracle.prefill_attention(q, k, v, cu, starts, True, 0.3)
    rows = [0, 7, 29, 30, 38]
    part, lp = oracle.prefill_attention(q, k, v, cu, starts, True, 0.3, rows=rows)
    np.testing.assert_allclose(part[rows], full[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lp[rows], lf[rows], rtol=0, atol=1e-13)
    assert np.all(part[1] == 0)


def test_prefill_last_row_equals_non_causal_row():
    q, k, v, cu, starts = _prefill_inputs(23, [25], 4, 1, 8)
    c, lc = oracle.prefill_attention(q, k, v, cu, starts, True, 0.3)
    nc, lnc = oracle.prefill_attention(q, k, v, cu, starts, False, 0.3)
    np.testing.assert_allclose(c[24], nc[24], rtol=0, atol=1e-13)
    assert not np.allclose(c[10], nc[10])


def test_prefill_row_equals_decode_over_prefix():
    """Row i of a prompt stored in compact pages with unit scales (so the
    unscaled gather workspace holds exactly the decode values) equals decode
    over the prompt's first i + 1 tokens."""
    rng = np.random.default_rng(31)
    n, hq, hkv, d = 37, 4, 2, 8
    keys = [rng.standard_normal((n, hkv, d)).astype(np.float16)]
    codes = [_fp8(rng.standard_normal((n, hkv, d)) * 30)]
    pages = (n + PAGE - 1) // PAGE
    scales = [np.ones((pages, hkv), np.float32)]
    pools = build_paged(rng, keys, [keys[0]], codes, scales, [[1] * pages])
    ids = pools["page_table"][0, :pages]
    ws_k, ws_v = oracle.gather_compact_pages(pools["k_compact"], pools["v_compact"], pools["v_scale"], ids, False)
    ws_k = ws_k.reshape(-1, hkv, d)
    ws_v = ws_v.reshape(-1, hkv, d)
    qp = rng.standard_normal((n, hq, d)).astype(np.float16)
    out_p, lse_p = oracle.prefill_attention(qp, ws_k, ws_v, [0, n], [0], True, 0.35)
    for i in (0, 15, 16, 36):
        pools["seq_lens"] = np.array([i + 1], np.int32)
        out_d, lse_d = _decode(qp[i:i + 1], pools, 0.35)
        np.testing.assert_allclose(out_p[i], out_d[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse_p[i], lse_d[0], rtol=0, atol=1e-13)

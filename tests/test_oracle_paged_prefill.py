"""Pins for the oracle's direct (workspace-free) paged prefill.

Pinned to torch scaled_dot_product_attention in float64 (library) on
contiguous tensors whose compact values are made with the library casts
(float8 -> float32, float32 multiply, float16), to page-permutation
invariance, and to the gather route composed from the oracle's own gather and
prefill (so the direct route and the gather route agree by construction only
if both are right).
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


def _prompts(seed, lens, hq, hkv, d, compact_prob):
    rng = np.random.default_rng(seed)
    keys, vals16, codes, scales, flags = [], [], [], [], []
    for n in lens:
        pages = (n + PAGE - 1) // PAGE
        keys.append(rng.standard_normal((n, hkv, d)).astype(np.float16))
        vals16.append(rng.standard_normal((n, hkv, d)).astype(np.float16))
        scales.append((rng.uniform(0.5, 2.0, size=(pages, hkv)) / 64).astype(np.float32))
        codes.append(_fp8(rng.standard_normal((n, hkv, d)) * 40))
        flags.append([int(rng.random() < compact_prob) for _ in range(pages)])
    pools = build_paged(rng, keys, vals16, codes, scales, flags)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), hq, d)).astype(np.float16)
    return q, cu, keys, vals16, codes, scales, flags, pools


def _library_values(vals16, codes, scales, flags):
    """fp16 values per token: TARGET as stored, compact = fp16(fp32(fp8) * fp32(scale)) via torch."""
    out = vals16.copy()
    for t in range(vals16.shape[0]):
        j = t // PAGE
        if flags[j]:
            v = torch.from_numpy(codes[t]).view(torch.float8_e4m3fn).to(torch.float32)
            out[t] = (v * torch.from_numpy(scales[j])[:, None]).to(torch.float16).numpy()
    return out


def _run(q, cu, pools, causal, sm, rows=None):
    return oracle.paged_prefill_attention(q, pools["k_target"], pools["v_target"], pools["k_compact"],
                                          pools["v_compact"], pools["v_scale"], pools["page_table"],
                                          pools["fidelity"], cu, causal, sm, rows=rows)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,d,prob", [(4, 1, 64, 0.5), (8, 2, 16, 1.0), (4, 2, 32, 0.0)])
def test_matches_sdpa_on_library_cast_values(causal, hq, hkv, d, prob):
    lens = [1, 17, 40, 33]
    q, cu, keys, vals16, codes, scales, flags, pools = _prompts(41, lens, hq, hkv, d, prob)
    sm = 1.0 / math.sqrt(d)
    out, lse = _run(q, cu, pools, causal, sm)
    for p, n in enumerate(lens):
        V = _library_values(vals16[p], codes[p], scales[p], flags[p])
        Q = torch.from_numpy(q[cu[p]:cu[p + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        K = torch.from_numpy(keys[p].astype(np.float64)).permute(1, 0, 2)[None]
        Vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(Q, K, Vt, is_causal=causal, scale=sm, enable_gqa=True)
        np.testing.assert_allclose(out[cu[p]:cu[p + 1]], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))   # NaN-poisoned slack never read


def test_page_permutation_invariant():
    lens = [50, 20]
    q, cu, keys, vals16, codes, scales, flags, pools = _prompts(42, lens, 4, 2, 16, 0.5)
    out, lse = _run(q, cu, pools, True, 0.25)
    rng = np.random.default_rng(5)
    for pool_key, kind in (("k_target", 0), ("k_compact", 1)):
        n_pool = pools[pool_key].shape[0]
        perm = rng.permutation(n_pool)            # new id of old page i is perm[i]
        moved = dict(pools)
        for name in (["k_target", "v_target"] if kind == 0 else ["k_compact", "v_compact", "v_scale"]):
            arr = pools[name].copy()
            arr[perm] = pools[name]
            moved[name] = arr
        table = pools["page_table"].copy()
        sel = pools["fidelity"] == kind
        table[sel] = perm[table[sel]]
        moved["page_table"] = table
        o2, l2 = _run(q, cu, moved, True, 0.25)
        np.testing.assert_array_equal(o2, out)
        np.testing.assert_array_equal(l2, lse)


def test_compact_prompts_equal_gather_route():
    lens = [64, 31]
    q, cu, keys, vals16, codes, scales, flags, pools = _prompts(43, lens, 4, 1, 32, 1.0)
    out, lse = _run(q, cu, pools, True, 0.2)
    ids = np.concatenate([pools["page_table"][p, :(n + 15) // 16] for p, n in enumerate(lens)])
    ws_k, ws_v = oracle.gather_compact_pages(pools["k_compact"], pools["v_compact"], pools["v_scale"], ids, True)
    kv_start = np.array([0, 64], np.int32)
    g_out, g_lse = oracle.prefill_attention(q, ws_k.reshape(-1, 1, 32), ws_v.reshape(-1, 1, 32), cu,
                                            kv_start, True, 0.2)
    np.testing.assert_array_equal(out, g_out)
    np.testing.assert_array_equal(lse, g_lse)


def test_unknown_flag_rejected():
    q, cu, keys, vals16, codes, scales, flags, pools = _prompts(44, [20], 4, 1, 16, 0.5)
    pools["fidelity"] = pools["fidelity"].copy()
    pools["fidelity"][0, 0] = 3
    with pytest.raises(ValueError):
        _run(q, cu, pools, True, 0.25)

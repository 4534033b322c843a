"""GPU parity: ElasticKV BASE pages — the demotion pack kernel (bit-exact) and decode over
TARGET / COMPACT / BASE pages in one launch, general (flag table) and structured
(TARGET-BASE-TARGET bounds) paths, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_close, assert_lse_close, dev, ekv, step
from mixed_precision_paged_amd import synth

pytestmark = pytest.mark.gpu


def _pools(case):
    t = dict(k_target=dev(case.k_target), v_target=dev(case.v_target))
    if case.k_compact.shape[0]:
        t.update(k_compact=dev(case.k_compact), v_compact=dev(case.v_compact), v_scale=dev(case.v_scale))
    return t


def _elastic_decode(case, structured_bounds=None, flags=True, has_base=True, pps=0):
    pools = _pools(case)
    kv = ekv().paged_kv(case.num_kv_heads, case.head_dim, **pools)
    out = torch.empty((case.batch, case.num_q_heads, case.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((case.batch, case.num_q_heads), dtype=torch.float32, device="cuda")
    ekv().ekv_decode_attention_elastic(
        kv, dev(case.q), dev(case.page_table), dev(case.fidelity) if flags else None,
        dev(structured_bounds) if structured_bounds is not None else None, has_base, dev(case.seq_lens),
        case.max_seq_len, case.sm_scale, out, lse, pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(case):
    return oracle.decode_attention(case.q, case.k_target, case.v_target, case.k_compact, case.v_compact,
                                   case.v_scale, case.page_table, case.fidelity, case.seq_lens, case.sm_scale)


def test_pack_pairs_bit_exact_in_place_and_skips():
    step("pack BASE pairs")
    rng = np.random.default_rng(60)
    for hkv, d in ((8, 128), (1, 64), (2, 64), (16, 128), (3, 64)):  # Hkv*D up to the 2048 limit
        n = 12
        k = synth.normal_fp16(rng, (n, 16, hkv, d))
        v = synth.normal_fp16(rng, (n, 16, hkv, d))
        src_a = np.array([0, 3, 6, 9, 1], np.int32)
        src_b = np.array([2, 4, 7, 10, n], np.int32)       # last pair: b out of the pool -> skipped
        dst = np.array([0, 4, 11, 9, 1], np.int32)         # in place on a, in place on b, elsewhere
        kt, vt = dev(k), dev(v)
        kv = ekv().paged_kv(hkv, d, kt, vt)
        ekv().ekv_pack_base_pairs(kv, dev(src_a), dev(src_b), dev(dst))
        torch.cuda.synchronize()
        wk, wv = oracle.pack_base_pairs(k, v, src_a[:4], src_b[:4], dst[:4])
        assert np.array_equal(kt.cpu().numpy().view(np.uint16), wk.view(np.uint16)), (hkv, d)
        assert np.array_equal(vt.cpu().numpy().view(np.uint16), wv.view(np.uint16)), (hkv, d)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 64), (16, 2, 128), (8, 1, 64), (16, 8, 128),
                                      (4, 2, 64)])
def test_general_path_target_compact_base_mix(hq, hkv, d):
    step(f"elastic decode, flag table, hq={hq} hkv={hkv} d={d}")
    e = synth.make_elastic_case(61 + d, [300, 1029, 64, 777, 16], hq, hkv, d, sink_pages=2, recent_pages=4,
                                structured=False, base_pair_frac=0.6, compact_frac=0.3)
    c = e.paged
    assert {0, 1, 2} <= set(np.unique(c.fidelity[c.page_table >= 0]).tolist())
    out, lse = _elastic_decode(c)
    want, wlse = _oracle(c)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


@pytest.mark.parametrize("d", [128, 64])
def test_structured_path_equals_general_path_and_oracle(d):
    step(f"elastic decode, structured bounds, d={d}")
    e = synth.make_elastic_case(70 + d, [2048, 333, 1500, 40, 4096], 32, 8, d, sink_pages=2, recent_pages=8)
    c = e.paged
    out_s, lse_s = _elastic_decode(c, structured_bounds=e.base_bounds, flags=False)
    out_g, lse_g = _elastic_decode(c)
    assert np.array_equal(out_s.view(np.uint32), out_g.view(np.uint32))
    assert np.array_equal(lse_s.view(np.uint32), lse_g.view(np.uint32))
    want, wlse = _oracle(c)
    assert_close(out_s, want)
    assert_lse_close(lse_s, wlse)


def test_split_plans_agree():
    step("elastic decode, split plans")
    e = synth.make_elastic_case(80, [3000, 2100, 700], 8, 2, 128, sink_pages=2, recent_pages=6)
    c = e.paged
    want, _ = _oracle(c)
    for pps in (16, 64, 512, ekv().DECODE_BALANCED):
        out, _ = _elastic_decode(c, structured_bounds=e.base_bounds, flags=False, pps=pps)
        assert_close(out, want, what=f"pages_per_split {pps}")
        out, _ = _elastic_decode(c, pps=pps)  # general path (flag table)
        assert_close(out, want, what=f"flags, pages_per_split {pps}")


def test_base_flags_without_indicator_are_invalid():
    """Without the batch-level BASE indicator a BASE flag is an unknown flag: NaN rows."""
    step("BASE flag without has_base")
    e = synth.make_elastic_case(81, [800, 64], 8, 2, 128, sink_pages=2, recent_pages=4)
    c = e.paged
    out, lse = _elastic_decode(c, has_base=False)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))     # sequence 0 has BASE pages
    want, _ = _oracle(c)
    assert_close(out[1:], want[1:])


def test_demote_with_pack_kernel_then_decode():
    """A TARGET batch demoted on the GPU (pairs packed in place) decodes like the oracle's
    pack + decode, and the freed blocks are never read (they are NaN-filled)."""
    step("pack kernel demotion, then elastic decode")
    c = synth.make_paged_case(82, [1024, 600], 16, 4, 128, compact_frac=0.0)
    pt, fl = c.page_table.copy(), c.fidelity.copy()
    src_a, src_b = [], []
    for b, n in enumerate(c.seq_lens):
        pages = int(n) // 16
        for j in range(2, pages - 4, 2):
            src_a.append(int(pt[b, j]))
            src_b.append(int(pt[b, j + 1]))
            pt[b, j], pt[b, j + 1] = 2 * pt[b, j], 2 * pt[b, j] + 1
            fl[b, j] = fl[b, j + 1] = 2
    src_a, src_b = np.array(src_a, np.int32), np.array(src_b, np.int32)
    kt, vt = dev(c.k_target), dev(c.v_target)
    kv = ekv().paged_kv(c.num_kv_heads, c.head_dim, kt, vt)
    ekv().ekv_pack_base_pairs(kv, dev(src_a), dev(src_b), dev(src_a))
    nan = torch.full((16, c.num_kv_heads, c.head_dim), float("nan"), dtype=torch.float16, device="cuda")
    for blk in src_b:
        kt[int(blk)] = nan
        vt[int(blk)] = nan
    out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((c.batch, c.num_q_heads), dtype=torch.float32, device="cuda")
    ekv().ekv_decode_attention_elastic(kv, dev(c.q), dev(pt), dev(fl), None, True, dev(c.seq_lens),
                                       c.max_seq_len, c.sm_scale, out, lse)
    torch.cuda.synchronize()
    wk, wv = oracle.pack_base_pairs(c.k_target, c.v_target, src_a, src_b, src_a)
    want, wlse = oracle.decode_attention(c.q, wk, wv, c.k_compact, c.v_compact, c.v_scale, pt, fl,
                                         c.seq_lens, c.sm_scale)
    assert_close(out.cpu().numpy(), want)
    assert_lse_close(lse.cpu().numpy(), wlse)


def test_bypass_and_forced_general_path_agree_on_target_batch():
    """A TARGET-only batch gives the same bits through the native path (indicator 0, no
    flags) and forced through the general elastic path (indicator 1, all-TARGET flags)."""
    step("bypass vs forced general path")
    c = synth.make_paged_case(83, [1500, 700, 3000], 16, 4, 128, compact_frac=0.0)
    out_n, lse_n = _elastic_decode(c, flags=False, has_base=False)
    out_g, lse_g = _elastic_decode(c, flags=True, has_base=True)
    assert np.array_equal(out_n.view(np.uint32), out_g.view(np.uint32))
    assert np.array_equal(lse_n.view(np.uint32), lse_g.view(np.uint32))
    want, wlse = _oracle(c)
    assert_close(out_n, want)

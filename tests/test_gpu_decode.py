"""GPU parity: mixed-fidelity paged decode vs the float64 oracle (max-abs <= 2e-3)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, DeviceCase, assert_close, assert_lse_close, dev, ekv,
                         f16_bits_equal_rne, max_abs, oracle_decode, step)
from mixed_precision_paged_amd import synth

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 37, 64, 300, 1000, 2053]


def test_tiny_decode_case():
    step("decode tiny")
    c = synth.tiny_decode_case()
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    out32, lse = dc.decode(torch.float32)
    assert_close(out32, want)
    assert_lse_close(lse, wlse)
    out16, _ = dc.decode(torch.float16)
    assert f16_bits_equal_rne(out16, out32)
    out_nf, _ = dc.decode(torch.float32, flags=False)  # uniform-pool path (no flag reads)
    np.testing.assert_array_equal(out_nf, out32)


# every (head dim, query heads per KV head) kernel instantiation: D 64 / 128 x G 1, 2, 4, 8
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 128), (16, 8, 128), (8, 1, 128),
                                      (8, 8, 64), (16, 8, 64), (8, 2, 64), (16, 2, 64)])
def test_mixed_fidelity_ragged(hq, hkv, d):
    step(f"decode mixed hq={hq} hkv={hkv} d={d}")
    c = synth.make_paged_case(100 + hq + d, LENS, hq, hkv, d, compact_frac=0.3,
                              outlier_frac=0.01, outlier_mult=20.0)
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    out, lse = dc.decode(torch.float32)
    assert_close(out, want)
    assert_lse_close(lse, wlse)


@pytest.mark.parametrize("frac", [0.0, 1.0])
def test_single_kind_batches(frac):
    step(f"decode single kind frac={frac}")
    c = synth.make_paged_case(7, LENS, 32, 8, 128, compact_frac=frac)
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    out, lse = dc.decode(torch.float32)
    assert_close(out, want)
    assert_lse_close(lse, wlse)
    out_nf, _ = dc.decode(torch.float32, flags=False)
    np.testing.assert_array_equal(out_nf, out)


def test_split_count_does_not_change_the_result():
    step("decode split counts")
    c = synth.make_paged_case(8, [2053, 700, 33], 32, 8, 128, compact_frac=0.5)
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    outs = []
    for pps in (1, 3, 16, 64, 0, 512, ekv().DECODE_BALANCED):
        out, lse = dc.decode(torch.float32, pages_per_split=pps)
        assert_close(out, want, what=f"pages_per_split={pps}")
        assert_lse_close(lse, wlse)
        outs.append(out)
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= TOL


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 2, 64), (8, 8, 128), (16, 2, 64), (16, 8, 64)])
def test_balanced_plan_ragged_empty_and_bad(hq, hkv, d):
    """Equal page-head shares per workgroup: sequences held whole by one range (1-page
    ones), cut over a few ranges and spread over hundreds (few page-heads, 256
    workgroups), empty ones, and a bad page id that must turn only its rows NaN."""
    step(f"decode balanced plan hq={hq} hkv={hkv} d={d}")
    lens = [1, 5, 16, 0, 17, 300, 2053, 40, 0, 1000, 3, 129, 64, 16, 777, 2]
    c = synth.make_paged_case(300 + d, lens, hq, hkv, d, compact_frac=0.4,
                              outlier_frac=0.01, outlier_mult=20.0)
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    out, lse = dc.decode(torch.float32, pages_per_split=ekv().DECODE_BALANCED)
    assert_close(out, want)
    assert_lse_close(lse, wlse)
    empty = np.array(lens) == 0
    assert np.all(out[empty] == 0) and np.all(np.isneginf(lse[empty]))
    out16, _ = dc.decode(torch.float16, pages_per_split=ekv().DECODE_BALANCED)
    assert f16_bits_equal_rne(out16, out)
    # a short batch: 37 + 1 tokens spread over 256 workgroups
    c2 = synth.make_paged_case(310 + d, [37, 1], hq, hkv, d, compact_frac=0.5)
    out2, lse2 = DeviceCase(c2).decode(torch.float32, pages_per_split=ekv().DECODE_BALANCED)
    w2, wl2 = oracle_decode(c2)
    assert_close(out2, w2)
    assert_lse_close(lse2, wl2)
    # every sequence empty, max_seq_len 0: out 0, lse -inf
    z = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    outz, lsez = dc.decode(torch.float32, pages_per_split=ekv().DECODE_BALANCED, seq_lens=z, max_seq_len=0)
    assert np.all(outz == 0) and np.all(np.isneginf(lsez))
    outz, lsez = dc.decode(torch.float32, seq_lens=z, max_seq_len=0)  # automatic plan
    assert np.all(outz == 0) and np.all(np.isneginf(lsez))
    # one bad page id in sequence 6 (2053 tokens, cut over several ranges)
    bad = c.page_table.copy()
    bad[6, 70] = 1 << 20
    dc.page_table = dev(bad)
    outb, lseb = dc.decode(torch.float32, pages_per_split=ekv().DECODE_BALANCED)
    assert np.all(np.isnan(outb[6])) and np.all(np.isnan(lseb[6]))
    keep = [i for i in range(len(lens)) if i != 6]
    assert_close(outb[keep], want[keep])


def test_one_split_plans_write_output_directly():
    """Automatic plans that give every (sequence, KV head) one split: 8-wavefront
    workgroups up to 256 groups, 4-wavefront ones from 512; the split kernel
    writes out / lse itself (no merge), including empty sequences."""
    for batch, lo, hi in ((32, 1, 4000), (64, 1, 200)):
        step(f"decode one-split plan batch={batch}")
        lens = np.random.default_rng(batch).integers(lo, hi, size=batch)
        lens[3] = 0
        c = synth.make_paged_case(400 + batch, lens, 32, 8, 128, compact_frac=0.5)
        assert ekv().ekv_decode_scratch_bytes(batch, 32, 8, 128, c.max_seq_len, 0) == 0
        dc = DeviceCase(c)
        want, wlse = oracle_decode(c)
        out, lse = dc.decode(torch.float32)
        assert_close(out, want)
        assert_lse_close(lse, wlse)
        assert np.all(out[3] == 0) and np.all(np.isneginf(lse[3]))
        out16, _ = dc.decode(torch.float16)
        assert f16_bits_equal_rne(out16, out)
        out_s, _ = dc.decode(torch.float32, pages_per_split=16)  # split + merge plan
        assert max_abs(out_s, out) <= TOL


def test_page_permutation_gives_identical_output():
    step("decode page permutation")
    c = synth.make_paged_case(9, [300, 129], 8, 2, 128, compact_frac=0.5, slack_frac=0.5)
    dc = DeviceCase(c)
    out1, lse1 = dc.decode(torch.float32, pages_per_split=4)
    # move every page to a new physical slot in both pools and rewrite the table
    rng = np.random.default_rng(1)
    c2 = synth.PagedCase(**{f: getattr(c, f) for f in c.__dataclass_fields__})
    pt = c.page_table.copy()
    for kind, names in ((0, ("k_target", "v_target")), (1, ("k_compact", "v_compact", "v_scale"))):
        P = getattr(c, names[0]).shape[0]
        perm = rng.permutation(P)
        inv = np.empty(P, np.int64)
        inv[perm] = np.arange(P)
        for n in names:
            setattr(c2, n, getattr(c, n)[perm])
        mask = c.fidelity == kind
        pt[mask] = inv[c.page_table[mask]]
    c2.page_table = pt
    assert not np.array_equal(pt, c.page_table)
    out2, lse2 = DeviceCase(c2).decode(torch.float32, pages_per_split=4)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_compact_page_with_exact_values_equals_target_page():
    step("decode compact==target")
    c = synth.make_paged_case(10, [200, 45], 8, 2, 64, compact_frac=1.0)
    # TARGET copy of every compact page with V = e4m3 value exactly (scale 1)
    c.v_scale[:] = 1.0
    vals = torch.from_numpy(c.v_compact).view(torch.float8_e4m3fn).to(torch.float16).numpy()
    ct = synth.PagedCase(**{f: getattr(c, f) for f in c.__dataclass_fields__})
    ct.k_target, ct.v_target = c.k_compact.copy(), vals
    ct.k_compact = c.k_compact[:0]
    ct.v_compact, ct.v_scale = c.v_compact[:0], c.v_scale[:0]
    ct.fidelity = np.zeros_like(c.fidelity)
    oc, lc = DeviceCase(c).decode(torch.float32)
    ot, lt = DeviceCase(ct).decode(torch.float32)
    np.testing.assert_array_equal(oc, ot)
    np.testing.assert_array_equal(lc, lt)


def test_empty_sequences_and_bad_pages():
    step("decode empty and bad pages")
    c = synth.make_paged_case(11, [40, 40, 40], 8, 2, 128, compact_frac=0.5)
    dc = DeviceCase(c)
    lens = c.seq_lens.copy()
    lens[1] = 0
    out, lse = dc.decode(torch.float32, seq_lens=dev(lens))
    want, wlse = oracle_decode(c, seq_lens=lens)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert_close(out[[0, 2]], want[[0, 2]])
    bad = c.page_table.copy()
    bad[2, 1] = 1 << 20  # out of range for either pool
    dc.page_table = dev(bad)
    out, lse = dc.decode(torch.float32)
    assert np.all(np.isnan(out[2])) and np.all(np.isnan(lse[2]))
    assert_close(out[:2], oracle_decode(c)[0][:2])
    badf = c.fidelity.copy()
    badf[0, 0] = 2
    dc.page_table, dc.fidelity = dev(c.page_table), dev(badf)
    out, _ = dc.decode(torch.float32)
    assert np.all(np.isnan(out[0])) and np.all(np.isfinite(out[1:]))


def test_planted_oracle_mistakes_are_detected():
    """Plant one wrong scale / page id / flag in the ORACLE's copy: parity must fail."""
    step("decode fault injection")
    c = synth.make_paged_case(12, [64, 64], 8, 2, 128, compact_frac=0.5)
    out, _ = DeviceCase(c).decode(torch.float32)
    assert max_abs(out, oracle_decode(c)[0]) <= TOL
    comp0 = np.flatnonzero(c.fidelity[0, :4] == 1)
    comp1 = np.flatnonzero(c.fidelity[1, :4] == 1)
    targ0 = np.flatnonzero(c.fidelity[0, :4] == 0)
    assert comp0.size and comp1.size and targ0.size
    sc = c.v_scale.copy()
    sc[c.page_table[0, comp0[0]]] *= 1.5                      # one wrong scale
    pt = c.page_table.copy()
    pt[0, comp0[0]], pt[1, comp1[0]] = pt[1, comp1[0]], pt[0, comp0[0]]  # two ids exchanged
    pt2, fl2 = c.page_table.copy(), c.fidelity.copy()
    pt2[0, targ0[0]], fl2[0, targ0[0]] = c.page_table[1, comp1[0]], 1   # one flag flipped
    for kwargs in (dict(v_scale=sc), dict(page_table=pt), dict(page_table=pt2, fidelity=fl2)):
        assert max_abs(out, oracle_decode(c, **kwargs)[0]) > TOL, list(kwargs)


def test_balanced_plan_at_its_batch_limit():
    """2,048 sequences (the balanced plan's largest batch: the page-count scan runs 32
    sequences per lane) of 0..300 tokens, mixed fidelity, 8 q / 2 KV heads, head dim 64;
    the automatic plan picks the balanced one for such a ragged batch."""
    step("decode balanced plan, 2048 sequences")
    lens = np.random.default_rng(2048).integers(0, 301, size=2048)
    assert ekv().ekv_decode_plan_pages_per_split(lens, 2) == ekv().DECODE_BALANCED
    c = synth.make_paged_case(2048, lens, 8, 2, 64, compact_frac=0.3)
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    out, lse = dc.decode(torch.float32, pages_per_split=ekv().DECODE_BALANCED)
    assert_close(out, want)
    assert_lse_close(lse, wlse)
    empty = lens == 0
    assert np.all(out[empty] == 0) and np.all(np.isneginf(lse[empty]))


def test_one_long_sequence_every_plan():
    """A 131,072-token sequence (8,192 pages) beside a 5-token one, mixed fidelity with
    value outliers, 32 q / 8 KV heads, head dim 128: the largest split counts (8,192
    one-page splits) and the longest balanced ranges still match the oracle, and every
    plan agrees with every other."""
    step("decode one long sequence, every plan")
    lens = [131072, 5]
    c = synth.make_paged_case(131072, lens, 32, 8, 128, compact_frac=0.3,
                              outlier_frac=0.01, outlier_mult=20.0)
    dc = DeviceCase(c)
    want, wlse = oracle_decode(c)
    host_plan = ekv().ekv_decode_plan_pages_per_split(np.asarray(lens), 8)
    outs = []
    for pps in (0, 1, 16, 512, ekv().DECODE_BALANCED, host_plan):
        out, lse = dc.decode(torch.float32, pages_per_split=pps)
        assert_close(out, want, what=f"pages_per_split={pps}")
        assert_lse_close(lse, wlse)
        outs.append(out)
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= TOL
    out16, _ = dc.decode(torch.float16)
    assert f16_bits_equal_rne(out16, outs[0])


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 2, 64)])
@pytest.mark.parametrize("scale_exp", [-13, -26, 14])
def test_compact_pages_with_extreme_page_scales(hq, hkv, d, scale_exp):
    """Compact page-head scales far from the ~2^-7 of N(0,1) data: the stored codes stay and
    the scales of sequence 0's pages (all of them), of every other page of sequence 1 and of
    no page of sequence 2 are multiplied by 2^scale_exp (scales near 2^-20 and 2^-33 -- the
    smallest a page of fp16 values can have -- and near 2^7).  Outputs against the oracle
    with the bound taken relative to each sequence's largest |V| (2e-3 at max|V| = 4), under
    the automatic plan, splits with a merge, and the balanced plan."""
    step(f"decode extreme page scales 2^{scale_exp} hq={hq} hkv={hkv} d={d}")
    c = synth.make_paged_case(70 + scale_exp + d, [700, 1000, 333], hq, hkv, d, compact_frac=1.0)
    f = np.float32(2.0 ** scale_exp)
    vs = c.v_scale.copy()
    for b, every in ((0, 1), (1, 2)):
        pages = c.page_table[b, :(int(c.seq_lens[b]) + 15) // 16][::every]
        vs[pages] = vs[pages] * f  # exact: power-of-two factor of normal fp32 values
    c.v_scale = vs
    want, wlse = oracle_decode(c)
    dc = DeviceCase(c)
    vmax = np.array([np.nanmax(np.abs(oracle.decode_e4m3fn(
        c.v_compact[c.page_table[b, :(int(c.seq_lens[b]) + 15) // 16]])) * vs[c.page_table[b, :(int(c.seq_lens[b]) + 15) // 16]][:, None, :, None])
        for b in range(c.batch)])
    for pps in (0, 16, ekv().DECODE_BALANCED):
        out, lse = dc.decode(torch.float32, pages_per_split=pps)
        assert np.all(np.isfinite(out)), pps
        for b in range(c.batch):
            err = np.abs(out[b].astype(np.float64) - want[b]).max()
            assert err <= TOL * vmax[b] / 4, (pps, b, err, vmax[b])
        assert_lse_close(lse, wlse)

"""Structure of the seeded synthetic inputs (no attention arithmetic here)."""
import numpy as np

from mixed_precision_paged_amd import synth


def test_tiny_case_pool_and_poison():
    c = synth.tiny_decode_case()
    assert c.k_compact.shape == (16, 16, 1, 64)
    assert list(c.seq_lens) == [37, 64]
    ids = np.concatenate([c.page_table[0, :3], c.page_table[1, :4]])
    assert len(set(ids.tolist())) == 7
    unused = sorted(set(range(16)) - set(ids.tolist()))
    assert len(unused) == 9
    assert np.all(np.isnan(c.k_compact[unused])) and np.all(c.v_compact[unused] == 0x7F)
    assert np.all(np.isnan(c.v_scale[unused]))
    last = c.page_table[0, 2]  # 37 = 2*16 + 5
    assert not np.any(np.isnan(c.k_compact[last, :5])) and np.all(np.isnan(c.k_compact[last, 5:]))
    assert np.all(c.v_compact[last, 5:] == 0x7F)
    assert np.all(c.fidelity[0, :3] == 1) and np.all(c.fidelity[1, :4] == 1)


def test_scale_is_absmax_over_448():
    import torch
    c = synth.make_paged_case(5, [20, 48], 4, 2, 16, compact_frac=1.0)
    vals = torch.from_numpy(c.v_compact).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for b in range(2):
        for j in range((c.seq_lens[b] + 15) // 16):
            p = c.page_table[b, j]
            n = min(16, c.seq_lens[b] - 16 * j)
            top = np.abs(vals[p, :n]).max(axis=(0, 2))
            np.testing.assert_array_equal(top, 448.0)  # absmax element maps to the largest code


def test_mixed_fraction_exact_and_pools_disjoint():
    c = synth.make_paged_case(9, [100, 333, 17], 8, 2, 16, compact_frac=0.3)
    pages = (c.seq_lens + 15) // 16
    owned = np.arange(c.page_table.shape[1])[None, :] < pages[:, None]
    n = int(owned.sum())
    assert int(c.fidelity[owned].sum()) == round(0.3 * n)
    for kind, pool in ((0, c.k_target), (1, c.k_compact)):
        ids = c.page_table[owned & (c.fidelity == kind)]
        assert len(set(ids.tolist())) == ids.size and ids.max() < pool.shape[0]


def test_deterministic():
    a = synth.make_paged_case(4, [40], 4, 1, 8, compact_frac=0.5)
    b = synth.make_paged_case(4, [40], 4, 1, 8, compact_frac=0.5)
    for f in ("q", "k_target", "v_compact", "page_table", "fidelity"):
        np.testing.assert_array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8))


def test_compact_decode_pool_size():
    assert synth._pool_size(16384, None, 0.0625) == 17408


def test_elastic_case_bounds_match_flags_and_pairs():
    """Structured layouts: flags are BASE exactly on [lo, hi) (pair-aligned, outside the
    protected sink and recent pages); a BASE pair (2i, 2i+1) names both halves of one block."""
    e = synth.make_elastic_case(3, [100, 600, 40, 333], 8, 2, 64, sink_pages=2, recent_pages=4)
    c = e.paged
    for b in range(c.batch):
        n = (int(c.seq_lens[b]) + 15) // 16
        lo, hi = (int(x) for x in e.base_bounds[b])
        want = np.zeros(n, np.uint8)
        want[lo:hi] = synth.BASE
        assert np.array_equal(c.fidelity[b, :n], want)
        assert lo % 2 == 0 and hi % 2 == 0 and (hi == 0 or (lo >= 2 and hi <= n - 4))
        for j in range(lo, hi, 2):
            assert c.page_table[b, j + 1] == c.page_table[b, j] + 1 and c.page_table[b, j] % 2 == 0

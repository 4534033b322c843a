"""The allocation-free decode entry point (ekv_decode_attention_noalloc), called
through the C ABI, against ekv_decode_attention on the same inputs: same plan and
kernels, so the outputs must be equal bit for bit (and within the oracle's bound).
Two calls in a row on the static scratch, the second with a smaller batch, so a
stale partial result of the first call would show in the second."""
import numpy as np
import pytest
import torch

from gpu_helpers import DeviceCase, assert_close, assert_lse_close, ekv, oracle_decode, step
from mixed_precision_paged_amd import synth

pytestmark = pytest.mark.gpu


def _both(dc, pps):
    c = dc.case
    shape = (c.batch, c.num_q_heads, c.head_dim)
    outs = []
    for fn in (ekv().ekv_decode_attention_noalloc, ekv().ekv_decode_attention):
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        fn(dc.kv(), dc.q, dc.page_table, dc.fidelity, dc.seq_lens, c.max_seq_len, c.sm_scale, out, lse,
           pages_per_split=pps)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    return outs


def test_noalloc_decode_matches_the_scratch_entry_point_on_two_calls():
    rng = np.random.default_rng(91)
    big = synth.make_paged_case(91, rng.integers(1, 3000, size=48), 32, 8, 128, compact_frac=0.3,
                                outlier_frac=0.01)
    small = synth.make_paged_case(92, rng.integers(1, 700, size=5), 32, 8, 128, compact_frac=0.5)
    for what, case, pps in (("48 ragged sequences, balanced plan", big, ekv().DECODE_BALANCED),
                            ("5 sequences, 16-page splits", small, 16)):
        need = ekv().ekv_decode_scratch_bytes(case.batch, 32, 8, 128, case.max_seq_len, pps)
        assert 0 < need <= ekv().NOALLOC_SCRATCH_BYTES, need
        step(f"noalloc decode: {what} ({need} scratch bytes)")
        (o_n, l_n), (o_s, l_s) = _both(DeviceCase(case), pps)
        assert np.array_equal(o_n.view(np.uint32), o_s.view(np.uint32)), what
        assert np.array_equal(l_n.view(np.uint32), l_s.view(np.uint32)), what
        want, wlse = oracle_decode(case)
        assert_close(o_n, want, what=what)
        assert_lse_close(l_n, wlse)


def test_noalloc_decode_refuses_a_plan_beyond_its_scratch():
    c = synth.tiny_decode_case()
    dc = DeviceCase(c)
    out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(ekv().EkvError) as e:  # 65,536-token bound with one-page splits
        ekv().ekv_decode_attention_noalloc(dc.kv(), dc.q, torch.zeros((2, 4096), dtype=torch.int32,
                                                                      device="cuda"),
                                           None, dc.seq_lens, 65536, c.sm_scale, out, pages_per_split=1)
    assert e.value.status == ekv().EKV_ERR_WORKSPACE_TOO_SMALL

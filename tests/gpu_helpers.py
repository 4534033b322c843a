"""Helpers for GPU parity tests: upload seeded cases, call the C ABI through
the Python binding, and compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = 2e-3  # max-abs bound on attention outputs and LSE (fp32 accumulation, N(0,1) inputs)


def step(msg: str) -> None:
    """Name the case before a GPU step, so a crash log says what ran."""
    print(f"[gpu-step] {msg}", flush=True)
    sys.stdout.flush()


def ekv():
    from mixed_precision_paged_amd import ekv as _ekv  # fails loudly if libekv.so is missing
    return _ekv


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


class DeviceCase:
    """A synth.PagedCase resident in device memory."""

    def __init__(self, case):
        self.case = case
        self.q = dev(case.q)
        self.k_target = dev(case.k_target) if case.k_target.shape[0] else None
        self.v_target = dev(case.v_target) if case.k_target.shape[0] else None
        self.k_compact = dev(case.k_compact) if case.k_compact.shape[0] else None
        self.v_compact = dev(case.v_compact) if case.k_compact.shape[0] else None
        self.v_scale = dev(case.v_scale) if case.k_compact.shape[0] else None
        self.page_table = dev(case.page_table)
        self.fidelity = dev(case.fidelity)
        self.seq_lens = dev(case.seq_lens)

    def kv(self):
        c = self.case
        return ekv().paged_kv(c.num_kv_heads, c.head_dim, self.k_target, self.v_target,
                              self.k_compact, self.v_compact, self.v_scale)

    def decode(self, out_dtype=torch.float32, pages_per_split=0, flags=True, q=None,
               rows=None, seq_lens=None, max_seq_len=None):
        c = self.case
        q = self.q if q is None else q
        pt = self.page_table if rows is None else self.page_table[rows].contiguous()
        fl = self.fidelity if rows is None else self.fidelity[rows].contiguous()
        sl = self.seq_lens if seq_lens is None else seq_lens
        B = q.shape[0]
        out = torch.empty((B, c.num_q_heads, c.head_dim), dtype=out_dtype, device="cuda")
        lse = torch.empty((B, c.num_q_heads), dtype=torch.float32, device="cuda")
        msl = c.max_seq_len if max_seq_len is None else max_seq_len
        ekv().ekv_decode_attention(self.kv(), q, pt, fl if flags else None, sl, msl, c.sm_scale,
                                   out, lse, pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()


def oracle_decode(case, q=None, seq_lens=None, page_table=None, fidelity=None, v_scale=None):
    return oracle.decode_attention(
        case.q if q is None else q, case.k_target, case.v_target, case.k_compact, case.v_compact,
        case.v_scale if v_scale is None else v_scale,
        case.page_table if page_table is None else page_table,
        case.fidelity if fidelity is None else fidelity,
        case.seq_lens if seq_lens is None else seq_lens, case.sm_scale)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    fin = np.isfinite(b)
    d = np.abs(a[fin] - b[fin])
    return float(d.max()) if d.size else 0.0


def assert_close(got, want, tol=TOL, what="output"):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.array_equal(np.isfinite(got), np.isfinite(want)) or np.all(np.isfinite(want)), what
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = max_abs(got, want)
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"
    return err


def assert_lse_close(got, want, tol=TOL):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    empty = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), empty), "lse: -inf pattern differs"
    err = float(np.abs(got[~empty] - want[~empty]).max()) if (~empty).any() else 0.0
    assert err <= tol, f"lse: max-abs error {err:.3e} > {tol:.1e}"
    return err


def f16_bits_equal_rne(out16: np.ndarray, out32: np.ndarray) -> bool:
    return np.array_equal(out16.view(np.uint16), out32.astype(np.float16).view(np.uint16))

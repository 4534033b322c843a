"""Byte/FLOP model pinned to the numbers the asymmetric-KV page prints."""
import json
import os

import numpy as np
import pytest

from mixed_precision_paged_amd import bytemodel

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "asym_byte_model.json")))


def test_bytes_per_pair_and_capacity():
    g = GOLD["bytes_per_pair"]
    for k in ("K16/V16", "K16/V8", "K8/V8"):
        assert bytemodel.BYTES_PER_PAIR[k] == g[k]
        cap = bytemodel.BYTES_PER_PAIR["K16/V16"] / bytemodel.BYTES_PER_PAIR[k]
        assert round(cap, 2) == g["capacity_vs_K16V16"][k]


def test_worked_bandwidth_example():
    w = GOLD["worked_example"]
    per_tok = bytemodel.kv_bytes_per_token(w["layers"], w["kv_heads"], w["head_dim"], "K16/V16")
    assert per_tok == w["bytes_per_token_K16V16_KiB"] * 1024
    for layout in ("K16/V16", "K16/V8", "K8/V8"):
        payload = bytemodel.kv_payload_bytes(w["tokens"], w["layers"], w["kv_heads"], w["head_dim"], layout)
        assert payload == w["payload_GiB"][layout] * 2 ** 30
        assert round(bytemodel.reread_gbps(payload, 0.010), 1) == w["reread_10ms_GBps"][layout]
        assert round(bytemodel.reread_gbps(payload, 1.0), 2) == w["reload_1s_GBps"][layout]


def test_token_slots_per_layer():
    s = GOLD["token_slots"]
    for layout in ("K16/V16", "K16/V8"):
        n = bytemodel.token_slots(s["pool_bytes"], s["layers"], s["kv_heads"], s["head_dim"], layout)
        assert n == s[layout]
        assert n * bytemodel.kv_bytes_per_token(s["layers"], s["kv_heads"], s["head_dim"], layout) == s["pool_bytes"]


def test_workspace_payload_size():
    w = GOLD["workspace"]
    _, written = bytemodel.gather_bytes(w["max_pages"], 8, 128)
    assert written == w["payload_MiB"] * 2 ** 20
    assert w["max_pages"] * 4 == w["indices_KiB"] * 1024


def test_decode_bytes_compact_batch():
    lens = [8192] * 32
    fid = np.ones((32, 512), np.uint8)
    b = bytemodel.decode_bytes(lens, fid, 32, 8, 128, out_bytes=2, flags_read=False)
    assert b == 805306368 + 524288 + 65536 + 262144 + 262144


def test_decode_bytes_counts_target_values_twice_and_partial_pages():
    fid = np.array([[0, 1, 0]], np.uint8)
    b = bytemodel.decode_bytes([40], fid, 2, 1, 4, out_bytes=4, lse=True)
    # tokens per page 16, 16, 8; K 2 B; V 2/1/2 B; one scale; ids + flags
    kv = 40 * 4 * 2 + (16 * 2 + 16 * 1 + 8 * 2) * 4
    assert b == kv + 4 + 3 * 5 + 2 * 4 * 2 + 2 * 4 * 4 + 2 * 4


def test_prefill_flops():
    assert bytemodel.prefill_flops([8192] * 32, 32, 128) == 32 * 2 * 128 * 32 * 8192 * 8193
    assert bytemodel.prefill_flops([3], 1, 1, causal=False) == 4 * 9


def test_writer_bytes_closed_forms():
    """Quantizer: 4 B read and 3 B written per K/V pair; the 32 x 8192 prompt set is
    16,384 full pages of 8 heads x 128 (268,435,456 pairs)."""
    pairs = 16384 * 16 * 8 * 128
    rd, wr = bytemodel.quantize_bytes(np.full(16384, 16), 8, 128)
    assert rd == 4 * pairs + 16384 * 12 == 1_073_938_432
    assert wr == 3 * pairs + 16384 * 8 * 4 == 805_830_656
    rd0, _ = bytemodel.quantize_bytes(np.full(16384, 16), 8, 128, n_valid_read=False)
    assert rd - rd0 == 16384 * 4
    # a partial page reads only its rows, but writes all 16 slots
    rd1, wr1 = bytemodel.quantize_bytes([5], 2, 64)
    assert rd1 == 5 * 2 * 64 * 4 + 12 and wr1 == 16 * 2 * 64 * 3 + 2 * 4
    assert bytemodel.append_bytes(32, 8, 128) == (32 * (4096 + 4), 32 * 4096)


def test_base_pages_move_half_the_target_bytes():
    """A BASE page moves 1 B of K and 1 B of V per element, no scale: half a TARGET page."""
    H, D = 8, 128
    lens = np.array([32])
    t = bytemodel.decode_bytes(lens, np.array([[0, 0]]), 32, H, D, flags_read=False)
    b = bytemodel.decode_bytes(lens, np.array([[2, 2]]), 32, H, D, flags_read=False)
    c = bytemodel.decode_bytes(lens, np.array([[1, 1]]), 32, H, D, flags_read=False)
    pairs = 32 * H * D
    assert t - b == 2 * pairs                     # 4 B vs 2 B per K/V pair
    assert c - b == pairs + 2 * H * 4             # 3 B vs 2 B per pair, plus the compact scales
    s = bytemodel.decode_bytes(lens, np.array([[2, 2]]), 32, H, D, flags_read=False, bounds_read=True)
    assert s - b == 8
    assert bytemodel.pack_bytes(10, H, D) == (10 * (4 * 16 * H * D * 2 + 12), 10 * 2 * 16 * H * D * 2)

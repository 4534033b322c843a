"""CPU oracle for mixed-fidelity paged-KV attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product path (the HIP library and its Python binding) never
calls it, and this package imports nothing from the product path: the two
share no kernels, helpers, tables or constants.  Inputs come from
``mixed_precision_paged_amd.synth`` (seeded generators, no attention
arithmetic) and are passed in as arrays.

Everything here is plain numpy float64 (plus the float32/float16 roundings
the gather contract names), written for a reader to check against the pages
by eye: no blocking, no fusion, no reordering.

Sources (page titles as published):
  [ekv]  "Does Execution Require Target KV Fidelity? A Mixed-Fidelity KV
         Runtime for LLM Serving" (ElasticKV).
  [asym] "Memory-Traffic Saturation in Autoregressive Transformer Decode"
         (asymmetric K16/V8 KV cache).

Pins: every function is pinned by tests under ``tests/test_oracle_*.py``
against closed forms, library routines (torch float8 casts, torch
scaled_dot_product_attention in float64) and invariants.  No function here
is "parity unpinned".
"""
from .e4m3 import E4M3FN_TABLE, e4m3fn_value, decode_e4m3fn
from .base import base_page, base_values, high_bytes, pack_base_pairs
from .paged import sequence_kv
from .attention import attention_rows, decode_attention, prefill_attention
from .gather import gather_compact_pages
from .paged_prefill import paged_prefill_attention, prompt_rows
from .writer import append_tokens, encode_e4m3fn, encode_e4m3fn_array, quantize_page, quantize_pages

__all__ = [
    "E4M3FN_TABLE", "e4m3fn_value", "decode_e4m3fn", "sequence_kv",
    "attention_rows", "decode_attention", "prefill_attention",
    "gather_compact_pages", "append_tokens", "quantize_page", "quantize_pages",
    "encode_e4m3fn", "encode_e4m3fn_array", "paged_prefill_attention", "prompt_rows",
    "base_page", "base_values", "high_bytes", "pack_base_pairs",
]

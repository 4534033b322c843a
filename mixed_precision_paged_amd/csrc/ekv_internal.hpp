// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ekv.h"

namespace ekv {

// Status helpers of the C ABI: `fail` records a thread-local message for
// ekv_last_error(), `ok` clears it, `hip_status` maps a HIP error.
ekv_status fail(ekv_status s, const char* fmt, ...);
ekv_status ok();
ekv_status hip_status(hipError_t e, const char* what);

// Argument checks, plan and launch of ekv_decode_attention(_elastic) with the
// scratch buffer given (shared by the allocation-free entry point).
ekv_status decode_entry(const ekv_paged_kv* kv, const void* q, int32_t batch, int32_t num_q_heads,
                        const int32_t* page_table, int32_t pt_stride, const uint8_t* fidelity,
                        const int32_t* base_bounds, int32_t has_base, const int32_t* seq_lens,
                        int32_t max_seq_len, float sm_scale, void* out, ekv_dtype out_dtype, float* lse,
                        int32_t pages_per_split, void* scratch, size_t scratch_bytes, void* stream);

struct DecodeParams {
  const uint16_t* k_target;
  const uint16_t* v_target;
  int32_t n_target;
  const uint16_t* k_compact;
  const uint8_t* v_compact;
  const float* v_scale;
  int32_t n_compact;
  const uint16_t* q;
  const int32_t* page_table;
  int32_t pt_stride;
  const uint8_t* fidelity;  // NULL: every page has kind `uniform_kind` (or base_bounds)
  int32_t uniform_kind;
  int32_t has_base;              // batch-level ElasticKV BASE indicator
  const int32_t* base_bounds;    // [batch][2] structured BASE range, when has_base and no flags
  const int32_t* seq_lens;
  int32_t batch, num_q_heads, num_kv_heads, head_dim, max_seq_len;
  int32_t pages_per_split, n_splits;
  int32_t n_wg;      // balanced plan: workgroups sharing all page-heads equally (0: split plan)
  float scale_log2;  // sm_scale * log2(e)
  float* part_acc;   // split plan [batch][Hkv][n_splits][G][D]; balanced [n_wg][2][G][D]
  float* part_ml;    // the same records' (max in log2 units, sum)
  void* out;
  int32_t out_f32;
  float* lse;
};

struct GatherParams {
  const uint16_t* k_compact;
  const uint8_t* v_compact;
  const float* v_scale;
  int32_t n_pool;
  const int32_t* page_ids;
  int32_t n_pages;
  int32_t num_kv_heads, head_dim;
  int32_t apply_scale;
  uint16_t* ws_k;
  uint16_t* ws_v;
};

struct PrefillParams {
  const uint16_t* q;
  int32_t q_rows;
  const uint16_t* k;
  const uint16_t* v;
  int32_t kv_rows;
  const int32_t* cu_seqlens_q;
  const int32_t* kv_start;
  int32_t n_prompts, max_len;
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t causal;
  float scale_log2;
  void* out;
  int32_t out_f32;
  float* lse;
  // Paged source (direct route): keys/values of prompt p come from its row of
  // page_table through the pools below; k, v, kv_start are unused then.
  const int32_t* page_table;  // [n_prompts][pt_stride]; NULL = workspace rows
  int32_t pt_stride;
  const uint8_t* fidelity;    // NULL: every page has kind uniform_kind
  int32_t uniform_kind;
  const uint16_t* k_target;
  const uint16_t* v_target;
  int32_t n_target;
  const uint16_t* k_compact;
  const uint8_t* v_compact;
  const float* v_scale;
  int32_t n_compact;
};

struct AppendParams {
  const uint16_t* k_new;        // [n_tokens][Hkv][D]
  const uint16_t* v_new;
  const int32_t* slot_mapping;  // [n_tokens], page * 16 + slot
  int64_t n_tokens;
  uint16_t* k_target;
  uint16_t* v_target;
  int32_t n_target;
  int32_t num_kv_heads, head_dim;
};

struct QuantizeParams {
  const uint16_t* k_src;        // [src_rows][Hkv][D]
  const uint16_t* v_src;
  int64_t src_rows;
  const int32_t* src_row_start;  // [n_pages]
  const int32_t* n_valid;        // [n_pages] or NULL (16 each)
  const int32_t* dst_pages;      // [n_pages]
  int32_t n_pages;
  uint16_t* k_compact;
  uint8_t* v_compact;
  float* v_scale;
  int32_t n_compact;
  int32_t num_kv_heads, head_dim;
};

struct PackParams {
  uint16_t* k_target;
  uint16_t* v_target;
  int32_t n_target;
  const int32_t* src_a;  // [n_pairs]
  const int32_t* src_b;
  const int32_t* dst;
  int32_t n_pairs;
  int32_t num_kv_heads, head_dim;
};

// Split plan shared by the scratch query and the launch.
int32_t decode_auto_pages_per_split(int32_t batch, int32_t num_kv_heads, int32_t max_pages);

size_t decode_scratch_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t n_splits);
// Balanced plan: workgroups for a batch whose longest sequence has max_pages
// pages, and the scratch bytes of their partial results.
constexpr int32_t kDecodeMaxBalancedBatch = 2048;
int32_t decode_balanced_workgroups(int32_t batch, int32_t num_kv_heads, int32_t max_pages);
size_t decode_balanced_scratch_bytes(int32_t n_wg, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim);

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream);
hipError_t launch_pack_base(const PackParams& p, hipStream_t stream);
hipError_t launch_e4m3_to_f16(const uint8_t* codes, int32_t n, uint16_t* out, int32_t method,
                              int32_t scale_exp, hipStream_t stream);

}  // namespace ekv

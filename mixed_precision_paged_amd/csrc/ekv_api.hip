// C ABI of libekv: argument validation, split planning, launches.
// Declarations and contracts: include/ekv.h.
#include "ekv.h"

#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "ekv_internal.hpp"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace ekv {

ekv_status fail(ekv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

ekv_status ok() {
  g_last_error[0] = '\0';
  return EKV_OK;
}

ekv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(EKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace ekv

namespace {

using ekv::fail;
using ekv::hip_status;
using ekv::ok;

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool supported_group(int32_t hq, int32_t hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv) return false;
  const int32_t g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

ekv_status check_geometry(int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0) return fail(EKV_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)", hq, hkv);
  if (hq % hkv) return fail(EKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", hq, hkv);
  if (!supported_group(hq, hkv)) return fail(EKV_ERR_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8}", hq / hkv);
  if (d != 64 && d != 128) return fail(EKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", d);
  return EKV_OK;
}

ekv_status check_kv(const ekv_paged_kv* kv, bool need_target, bool need_compact) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  if (kv->page_size != EKV_PAGE_SIZE) return fail(EKV_ERR_INVALID_ARG, "page_size %d != %d", kv->page_size, EKV_PAGE_SIZE);
  if (kv->n_target_pages < 0 || kv->n_compact_pages < 0) return fail(EKV_ERR_INVALID_ARG, "negative pool size");
  if (kv->n_target_pages >= (1 << 28) || kv->n_compact_pages >= (1 << 28))
    return fail(EKV_ERR_UNSUPPORTED, "pools of 2^28 pages or more are not supported");
  if (need_target || kv->n_target_pages > 0) {
    if (!kv->k_target || !kv->v_target) return fail(EKV_ERR_INVALID_ARG, "target pool pointer is NULL");
    if (!aligned16(kv->k_target) || !aligned16(kv->v_target)) return fail(EKV_ERR_INVALID_ARG, "target pool not 16-byte aligned");
  }
  if (need_compact || kv->n_compact_pages > 0) {
    if (!kv->k_compact || !kv->v_compact || !kv->v_scale) return fail(EKV_ERR_INVALID_ARG, "compact pool pointer is NULL");
    if (!aligned16(kv->k_compact) || !aligned16(kv->v_compact)) return fail(EKV_ERR_INVALID_ARG, "compact pool not 16-byte aligned");
  }
  return EKV_OK;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// 4-wavefront split-plan decode workgroups resident at once on the 256-CU
// part (3 per CU at their register use).
constexpr int64_t kSplitRound = 768;

}  // namespace

extern "C" {

int32_t ekv_abi_version(void) { return EKV_ABI_VERSION; }

#ifndef EKV_BUILD_ID
#define EKV_BUILD_ID "unknown"
#endif
const char* ekv_build_id(void) { return EKV_BUILD_ID; }

const char* ekv_status_string(ekv_status s) {
  switch (s) {
    case EKV_OK: return "ok";
    case EKV_ERR_INVALID_ARG: return "invalid argument";
    case EKV_ERR_UNSUPPORTED: return "unsupported shape";
    case EKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case EKV_ERR_NOT_ELIGIBLE: return "not eligible for the compact prefill route";
    case EKV_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* ekv_last_error(void) { return g_last_error; }

int32_t ekv_decode_pages_per_split(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  if (batch <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return 16;
  return ekv::decode_auto_pages_per_split(batch, num_kv_heads, ceil_div(max_seq_len, EKV_PAGE_SIZE));
}

int32_t ekv_decode_plan_pages_per_split(const int32_t* seq_lens_host, int32_t batch,
                                        int32_t num_kv_heads) {
  if (!seq_lens_host || batch <= 0 || num_kv_heads <= 0) return 16;
  int64_t total = 0, maxp = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = seq_lens_host[b] > 0 ? (seq_lens_host[b] + EKV_PAGE_SIZE - 1) / EKV_PAGE_SIZE : 0;
    total += n;
    maxp = n > maxp ? n : maxp;
  }
  if (maxp == 0) return 16;
  if (total * 10 >= maxp * batch * 9) {  // lengths within ~10% of the longest: splits
    const int32_t pps = ekv::decode_auto_pages_per_split(batch, num_kv_heads, (int32_t)maxp);
    // ... unless the split plan launches more than one round of its
    // 4-wavefront workgroups (768 resident on the 256-CU part at 3 per CU),
    // or only a few long sequences.  Equal shares measured ahead there, the
    // splits everywhere else (us, splits vs equal shares, V loads
    // non-temporal): one to two rounds, batch 128 x 8192 tokens 528 both,
    // 32 x 32768 526 both, 128 x 2048 148 vs 146; more rounds, 64 x 32768
    // 1068 vs 1032, 128 x 32768 2075 vs 2008; at most 32 (sequence, KV head)
    // groups of 2,048+ pages, 1 x 32768 37.8 vs 32.2, 4 x 32768 70.2 vs 68.1;
    // one round or less, 64 x 8192 261 vs 269, 16 x 32768 264 vs 269.
    const int64_t groups = (int64_t)batch * num_kv_heads;
    const int64_t wgs = groups * ((maxp + pps - 1) / pps);
    const bool eight_wave = groups <= 256 && wgs == groups;
    if (batch <= ekv::kDecodeMaxBalancedBatch &&
        ((!eight_wave && wgs > kSplitRound) || (groups <= 32 && maxp >= 2048)))
      return EKV_DECODE_BALANCED;
    return pps;
  }
  // ragged lengths: equal shares of all page-heads per workgroup
  if (batch <= ekv::kDecodeMaxBalancedBatch) return EKV_DECODE_BALANCED;
  int64_t c = (total * num_kv_heads + 4095) / 4096;  // else small splits balance the tail
  c = (c + 3) / 4 * 4;
  return (int32_t)(c < 16 ? 16 : (c > 512 ? 512 : c));
}

size_t ekv_decode_scratch_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_seq_len, int32_t pages_per_split) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0) return 0;
  if (pages_per_split == EKV_DECODE_BALANCED) {  // also for max_seq_len 0 (the merge writes empty rows)
    if (num_q_heads % num_kv_heads != 0) return 0;
    const int32_t n = ekv::decode_balanced_workgroups(batch, num_kv_heads, ceil_div(max_seq_len, EKV_PAGE_SIZE));
    return ekv::decode_balanced_scratch_bytes(n, num_q_heads, num_kv_heads, head_dim);
  }
  if (max_seq_len == 0) return 0;
  const int32_t pps = pages_per_split > 0 ? pages_per_split
                                          : ekv_decode_pages_per_split(batch, num_kv_heads, max_seq_len);
  const int32_t splits = ceil_div(ceil_div(max_seq_len, EKV_PAGE_SIZE), pps);
  return ekv::decode_scratch_bytes(batch, num_q_heads, num_kv_heads, head_dim, splits);
}

}  // extern "C"

namespace ekv {

ekv_status decode_entry(const ekv_paged_kv* kv, const void* q, int32_t batch, int32_t num_q_heads,
                        const int32_t* page_table, int32_t pt_stride, const uint8_t* fidelity,
                        const int32_t* base_bounds, int32_t has_base, const int32_t* seq_lens,
                        int32_t max_seq_len, float sm_scale, void* out, ekv_dtype out_dtype, float* lse,
                        int32_t pages_per_split, void* scratch, size_t scratch_bytes, void* stream) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  ekv_status s = check_geometry(num_q_heads, kv->num_kv_heads, kv->head_dim);
  if (s != EKV_OK) return s;
  s = check_kv(kv, false, false);
  if (s != EKV_OK) return s;
  if (batch < 0) return fail(EKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (max_seq_len < 0) return fail(EKV_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if (batch == 0) return ok();
  if (!q || !page_table || !seq_lens || !out) return fail(EKV_ERR_INVALID_ARG, "q, page_table, seq_lens and out are required");
  if (!aligned16(q)) return fail(EKV_ERR_INVALID_ARG, "q not 16-byte aligned");
  if (out_dtype != EKV_F16 && out_dtype != EKV_F32) return fail(EKV_ERR_INVALID_ARG, "out_dtype %d unknown", (int)out_dtype);
  if (!std::isfinite(sm_scale)) return fail(EKV_ERR_INVALID_ARG, "sm_scale is not finite");
  const int32_t max_pages = ceil_div(max_seq_len, EKV_PAGE_SIZE);
  if (pt_stride < max_pages || pt_stride <= 0) return fail(EKV_ERR_INVALID_ARG, "pt_stride %d < ceil(max_seq_len/16) = %d", pt_stride, max_pages);
  const bool has_t = kv->n_target_pages > 0, has_c = kv->n_compact_pages > 0;
  int32_t uniform_kind = 0;
  if (has_base != 0 && has_base != 1) return fail(EKV_ERR_INVALID_ARG, "has_base must be 0 or 1");
  if (!has_base && base_bounds) return fail(EKV_ERR_INVALID_ARG, "base_bounds needs has_base = 1");
  if (has_base) {
    if (!has_t) return fail(EKV_ERR_INVALID_ARG, "BASE pages live in the TARGET pool, which is empty");
    if (!fidelity && !base_bounds) return fail(EKV_ERR_INVALID_ARG, "has_base needs fidelity flags or base_bounds");
    if (fidelity && base_bounds) return fail(EKV_ERR_INVALID_ARG, "give fidelity flags or base_bounds, not both");
  } else if (!fidelity) {
    if (has_t == has_c) return fail(EKV_ERR_INVALID_ARG, "fidelity may be NULL only when exactly one pool is non-empty");
    uniform_kind = has_c ? EKV_FIDELITY_COMPACT : EKV_FIDELITY_TARGET;
  }
  const bool balanced = pages_per_split == EKV_DECODE_BALANCED;
  if (!balanced && (pages_per_split < 0 || pages_per_split > 512))
    return fail(EKV_ERR_INVALID_ARG, "pages_per_split %d outside 0..512 and not EKV_DECODE_BALANCED", pages_per_split);
  if (balanced && batch > ekv::kDecodeMaxBalancedBatch)
    return fail(EKV_ERR_UNSUPPORTED, "balanced plan takes at most %d sequences", ekv::kDecodeMaxBalancedBatch);
  const int32_t pps = balanced ? 0
                      : pages_per_split > 0 ? pages_per_split
                                            : ekv_decode_pages_per_split(batch, kv->num_kv_heads, max_seq_len);
  const int32_t splits = balanced ? 0 : max_pages > 0 ? ceil_div(max_pages, pps) : 0;
  const int32_t n_wg = balanced ? ekv::decode_balanced_workgroups(batch, kv->num_kv_heads, max_pages) : 0;
  const size_t need = balanced ? ekv::decode_balanced_scratch_bytes(n_wg, num_q_heads, kv->num_kv_heads, kv->head_dim)
                               : ekv::decode_scratch_bytes(batch, num_q_heads, kv->num_kv_heads, kv->head_dim, splits);
  if (need > 0) {  // more than one split: partial results go through scratch
    if (!scratch) return fail(EKV_ERR_INVALID_ARG, "scratch is NULL (%zu bytes needed)", need);
    if (((uintptr_t)scratch & 255u) != 0) return fail(EKV_ERR_INVALID_ARG, "scratch not 256-byte aligned");
    if (scratch_bytes < need) return fail(EKV_ERR_INVALID_ARG, "scratch of %zu bytes < %zu needed", scratch_bytes, need);
  }
  if ((int64_t)batch * num_q_heads > 65535LL * 65535LL || batch > 65535 || splits > 65535)
    return fail(EKV_ERR_UNSUPPORTED, "launch grid too large");

  ekv::DecodeParams p{};
  p.k_target = static_cast<const uint16_t*>(kv->k_target);
  p.v_target = static_cast<const uint16_t*>(kv->v_target);
  p.n_target = kv->n_target_pages;
  p.k_compact = static_cast<const uint16_t*>(kv->k_compact);
  p.v_compact = kv->v_compact;
  p.v_scale = kv->v_scale;
  p.n_compact = kv->n_compact_pages;
  p.q = static_cast<const uint16_t*>(q);
  p.page_table = page_table;
  p.pt_stride = pt_stride;
  p.fidelity = fidelity;
  p.uniform_kind = uniform_kind;
  p.has_base = has_base;
  p.base_bounds = base_bounds;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  p.max_seq_len = max_seq_len;
  p.pages_per_split = pps;
  p.n_splits = splits;
  p.n_wg = n_wg;  // balanced plan (also when every sequence is empty: its merge writes them)
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  const size_t rows = balanced ? (size_t)n_wg * 2 * (num_q_heads / kv->num_kv_heads)
                               : (size_t)batch * num_q_heads * (size_t)splits;
  p.part_acc = need > 0 ? static_cast<float*>(scratch) : nullptr;
  p.part_ml = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(scratch) +
                                                    ((rows * kv->head_dim * sizeof(float) + 255) & ~(size_t)255))
                         : nullptr;
  p.out = out;
  p.out_f32 = out_dtype == EKV_F32;
  p.lse = lse;
  return hip_status(ekv::launch_decode(p, static_cast<hipStream_t>(stream)), "decode launch");
}

}  // namespace ekv

extern "C" {

ekv_status ekv_decode_attention(const ekv_paged_kv* kv, const void* q, int32_t batch,
                                int32_t num_q_heads, const int32_t* page_table, int32_t pt_stride,
                                const uint8_t* fidelity, const int32_t* seq_lens,
                                int32_t max_seq_len, float sm_scale, void* out, ekv_dtype out_dtype,
                                float* lse, int32_t pages_per_split, void* scratch,
                                size_t scratch_bytes, void* stream) {
  return ekv::decode_entry(kv, q, batch, num_q_heads, page_table, pt_stride, fidelity, nullptr, 0, seq_lens,
                     max_seq_len, sm_scale, out, out_dtype, lse, pages_per_split, scratch, scratch_bytes,
                     stream);
}

ekv_status ekv_decode_attention_elastic(const ekv_paged_kv* kv, const void* q, int32_t batch,
                                        int32_t num_q_heads, const int32_t* page_table,
                                        int32_t pt_stride, const uint8_t* fidelity,
                                        const int32_t* base_bounds, int32_t has_base,
                                        const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                        void* out, ekv_dtype out_dtype, float* lse,
                                        int32_t pages_per_split, void* scratch, size_t scratch_bytes,
                                        void* stream) {
  return ekv::decode_entry(kv, q, batch, num_q_heads, page_table, pt_stride, fidelity, base_bounds, has_base,
                     seq_lens, max_seq_len, sm_scale, out, out_dtype, lse, pages_per_split, scratch,
                     scratch_bytes, stream);
}

ekv_status ekv_gather_compact_pages(const ekv_paged_kv* kv, const int32_t* page_ids,
                                    int32_t n_pages, int32_t apply_scale, void* ws_k, void* ws_v,
                                    int32_t ws_capacity_pages, void* stream) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  if (kv->head_dim != 64 && kv->head_dim != 128) return fail(EKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", kv->head_dim);
  if (kv->num_kv_heads <= 0) return fail(EKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
  ekv_status s = check_kv(kv, false, true);
  if (s != EKV_OK) return s;
  if (n_pages < 0 || ws_capacity_pages < 0) return fail(EKV_ERR_INVALID_ARG, "negative page count");
  if (n_pages > ws_capacity_pages)
    return fail(EKV_ERR_WORKSPACE_TOO_SMALL, "%d pages do not fit a workspace of %d pages", n_pages, ws_capacity_pages);
  if (apply_scale != 0 && apply_scale != 1) return fail(EKV_ERR_INVALID_ARG, "apply_scale must be 0 or 1");
  if (n_pages == 0) return ok();
  if (!page_ids || !ws_k || !ws_v) return fail(EKV_ERR_INVALID_ARG, "page_ids, ws_k and ws_v are required");
  if (!aligned16(ws_k) || !aligned16(ws_v)) return fail(EKV_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  ekv::GatherParams p{};
  p.k_compact = static_cast<const uint16_t*>(kv->k_compact);
  p.v_compact = kv->v_compact;
  p.v_scale = kv->v_scale;
  p.n_pool = kv->n_compact_pages;
  p.page_ids = page_ids;
  p.n_pages = n_pages;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  p.apply_scale = apply_scale;
  p.ws_k = static_cast<uint16_t*>(ws_k);
  p.ws_v = static_cast<uint16_t*>(ws_v);
  return hip_status(ekv::launch_gather(p, static_cast<hipStream_t>(stream)), "gather launch");
}

ekv_status ekv_prefill_attention(const void* q, int32_t q_rows, const void* k, const void* v,
                                 int32_t kv_rows, const int32_t* cu_seqlens_q,
                                 const int32_t* kv_start, int32_t n_prompts, int32_t max_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t causal, float sm_scale, void* out, ekv_dtype out_dtype,
                                 float* lse, void* stream) {
  ekv_status s = check_geometry(num_q_heads, num_kv_heads, head_dim);
  if (s != EKV_OK) return s;
  if (n_prompts < 0 || max_len < 0 || q_rows < 0 || kv_rows < 0) return fail(EKV_ERR_INVALID_ARG, "negative size");
  if (max_len > EKV_MAX_PREFILL_TOKENS)
    return fail(EKV_ERR_NOT_ELIGIBLE, "prompt bound %d exceeds %d tokens", max_len, EKV_MAX_PREFILL_TOKENS);
  if (causal != 0 && causal != 1) return fail(EKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (out_dtype != EKV_F16 && out_dtype != EKV_F32) return fail(EKV_ERR_INVALID_ARG, "out_dtype %d unknown", (int)out_dtype);
  // the prefill kernels take a row's max before scaling and mask before scaling
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(EKV_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (n_prompts == 0 || max_len == 0) return ok();
  if (!q || !k || !v || !cu_seqlens_q || !kv_start || !out)
    return fail(EKV_ERR_INVALID_ARG, "q, k, v, cu_seqlens_q, kv_start and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(EKV_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  const int64_t tiles = (int64_t)((max_len + 127) / 128) * num_q_heads * n_prompts;
  if (tiles > 0x7FFFFFFFLL) return fail(EKV_ERR_UNSUPPORTED, "launch grid too large");
  ekv::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_rows = q_rows;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kv_rows = kv_rows;
  p.cu_seqlens_q = cu_seqlens_q;
  p.kv_start = kv_start;
  p.n_prompts = n_prompts;
  p.max_len = max_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.causal = causal;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.out = out;
  p.out_f32 = out_dtype == EKV_F32;
  p.lse = lse;
  return hip_status(ekv::launch_prefill(p, static_cast<hipStream_t>(stream)), "prefill launch");
}

ekv_status ekv_prefill_paged_attention(const ekv_paged_kv* kv, const void* q, int32_t q_rows,
                                       const int32_t* cu_seqlens_q, const int32_t* page_table,
                                       int32_t pt_stride, const uint8_t* fidelity, int32_t n_prompts,
                                       int32_t max_len, int32_t num_q_heads, int32_t causal,
                                       float sm_scale, void* out, ekv_dtype out_dtype, float* lse,
                                       void* stream) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  ekv_status s = check_geometry(num_q_heads, kv->num_kv_heads, kv->head_dim);
  if (s != EKV_OK) return s;
  s = check_kv(kv, false, false);
  if (s != EKV_OK) return s;
  if (n_prompts < 0 || max_len < 0 || q_rows < 0) return fail(EKV_ERR_INVALID_ARG, "negative size");
  if (max_len > EKV_MAX_PREFILL_TOKENS)
    return fail(EKV_ERR_NOT_ELIGIBLE, "prompt bound %d exceeds %d tokens", max_len, EKV_MAX_PREFILL_TOKENS);
  if (causal != 0 && causal != 1) return fail(EKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (out_dtype != EKV_F16 && out_dtype != EKV_F32) return fail(EKV_ERR_INVALID_ARG, "out_dtype %d unknown", (int)out_dtype);
  // the prefill kernels take a row's max before scaling and mask before scaling
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(EKV_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (n_prompts == 0 || max_len == 0) return ok();
  if (!q || !cu_seqlens_q || !page_table || !out)
    return fail(EKV_ERR_INVALID_ARG, "q, cu_seqlens_q, page_table and out are required");
  if (!aligned16(q) || !aligned16(out)) return fail(EKV_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (pt_stride < ceil_div(max_len, EKV_PAGE_SIZE))
    return fail(EKV_ERR_INVALID_ARG, "pt_stride %d < ceil(max_len/16) = %d", pt_stride, ceil_div(max_len, EKV_PAGE_SIZE));
  const bool has_t = kv->n_target_pages > 0, has_c = kv->n_compact_pages > 0;
  int32_t uniform_kind = 0;
  if (!fidelity) {
    if (has_t == has_c) return fail(EKV_ERR_INVALID_ARG, "fidelity may be NULL only when exactly one pool is non-empty");
    uniform_kind = has_c ? EKV_FIDELITY_COMPACT : EKV_FIDELITY_TARGET;
  }
  const int64_t tiles = (int64_t)((max_len + 127) / 128) * num_q_heads * n_prompts;
  if (tiles > 0x7FFFFFFFLL) return fail(EKV_ERR_UNSUPPORTED, "launch grid too large");
  ekv::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_rows = q_rows;
  p.cu_seqlens_q = cu_seqlens_q;
  p.n_prompts = n_prompts;
  p.max_len = max_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  p.causal = causal;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.out = out;
  p.out_f32 = out_dtype == EKV_F32;
  p.lse = lse;
  p.page_table = page_table;
  p.pt_stride = pt_stride;
  p.fidelity = fidelity;
  p.uniform_kind = uniform_kind;
  p.k_target = static_cast<const uint16_t*>(kv->k_target);
  p.v_target = static_cast<const uint16_t*>(kv->v_target);
  p.n_target = kv->n_target_pages;
  p.k_compact = static_cast<const uint16_t*>(kv->k_compact);
  p.v_compact = kv->v_compact;
  p.v_scale = kv->v_scale;
  p.n_compact = kv->n_compact_pages;
  return hip_status(ekv::launch_prefill(p, static_cast<hipStream_t>(stream)), "paged prefill launch");
}

ekv_status ekv_append_tokens(const ekv_paged_kv* kv, const void* k_new, const void* v_new,
                             const int32_t* slot_mapping, int32_t n_tokens, void* stream) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  if (kv->head_dim != 64 && kv->head_dim != 128) return fail(EKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", kv->head_dim);
  if (kv->num_kv_heads <= 0) return fail(EKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
  ekv_status s = check_kv(kv, true, false);
  if (s != EKV_OK) return s;
  if ((int64_t)kv->n_target_pages * EKV_PAGE_SIZE > 0x7FFFFFFFLL)
    return fail(EKV_ERR_UNSUPPORTED, "target pool of %d pages exceeds int32 slot numbers", kv->n_target_pages);
  if (n_tokens < 0) return fail(EKV_ERR_INVALID_ARG, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return ok();
  if (!k_new || !v_new || !slot_mapping) return fail(EKV_ERR_INVALID_ARG, "k_new, v_new and slot_mapping are required");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(EKV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  ekv::AppendParams p{};
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.slot_mapping = slot_mapping;
  p.n_tokens = n_tokens;
  p.k_target = static_cast<uint16_t*>(const_cast<void*>(kv->k_target));
  p.v_target = static_cast<uint16_t*>(const_cast<void*>(kv->v_target));
  p.n_target = kv->n_target_pages;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  return hip_status(ekv::launch_append(p, static_cast<hipStream_t>(stream)), "append launch");
}

ekv_status ekv_quantize_pages(const ekv_paged_kv* kv, const void* k_src, const void* v_src,
                              int64_t src_rows, const int32_t* src_row_start,
                              const int32_t* n_valid, const int32_t* dst_pages, int32_t n_pages,
                              void* stream) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  if (kv->head_dim != 64 && kv->head_dim != 128) return fail(EKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", kv->head_dim);
  if (kv->num_kv_heads <= 0) return fail(EKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
  if ((int64_t)kv->num_kv_heads * kv->head_dim * 2 * EKV_PAGE_SIZE > 0x7FFFFFFFLL)
    return fail(EKV_ERR_UNSUPPORTED, "page of %d KV heads too large", kv->num_kv_heads);
  ekv_status s = check_kv(kv, false, true);
  if (s != EKV_OK) return s;
  if (n_pages < 0 || src_rows < 0) return fail(EKV_ERR_INVALID_ARG, "negative size");
  if (n_pages == 0) return ok();
  if (!k_src || !v_src || !src_row_start || !dst_pages)
    return fail(EKV_ERR_INVALID_ARG, "k_src, v_src, src_row_start and dst_pages are required");
  if (!aligned16(k_src) || !aligned16(v_src)) return fail(EKV_ERR_INVALID_ARG, "k_src and v_src must be 16-byte aligned");
  ekv::QuantizeParams p{};
  p.k_src = static_cast<const uint16_t*>(k_src);
  p.v_src = static_cast<const uint16_t*>(v_src);
  p.src_rows = src_rows;
  p.src_row_start = src_row_start;
  p.n_valid = n_valid;
  p.dst_pages = dst_pages;
  p.n_pages = n_pages;
  p.k_compact = static_cast<uint16_t*>(const_cast<void*>(kv->k_compact));
  p.v_compact = const_cast<uint8_t*>(kv->v_compact);
  p.v_scale = const_cast<float*>(kv->v_scale);
  p.n_compact = kv->n_compact_pages;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  return hip_status(ekv::launch_quantize(p, static_cast<hipStream_t>(stream)), "quantize launch");
}

ekv_status ekv_pack_base_pairs(const ekv_paged_kv* kv, const int32_t* src_a, const int32_t* src_b,
                               const int32_t* dst, int32_t n_pairs, void* stream) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv descriptor is NULL");
  if (kv->head_dim != 64 && kv->head_dim != 128) return fail(EKV_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", kv->head_dim);
  if (kv->num_kv_heads <= 0) return fail(EKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
  if ((int64_t)kv->num_kv_heads * kv->head_dim > 2048)
    return fail(EKV_ERR_UNSUPPORTED, "num_kv_heads * head_dim = %d exceeds 2048", kv->num_kv_heads * kv->head_dim);
  ekv_status s = check_kv(kv, true, false);
  if (s != EKV_OK) return s;
  if (n_pairs < 0) return fail(EKV_ERR_INVALID_ARG, "n_pairs %d < 0", n_pairs);
  if (n_pairs == 0) return ok();
  if (n_pairs > 0x7FFFFFFF / 2) return fail(EKV_ERR_UNSUPPORTED, "too many pairs");
  if (!src_a || !src_b || !dst) return fail(EKV_ERR_INVALID_ARG, "src_a, src_b and dst are required");
  ekv::PackParams p{};
  p.k_target = static_cast<uint16_t*>(const_cast<void*>(kv->k_target));
  p.v_target = static_cast<uint16_t*>(const_cast<void*>(kv->v_target));
  p.n_target = kv->n_target_pages;
  p.src_a = src_a;
  p.src_b = src_b;
  p.dst = dst;
  p.n_pairs = n_pairs;
  p.num_kv_heads = kv->num_kv_heads;
  p.head_dim = kv->head_dim;
  return hip_status(ekv::launch_pack_base(p, static_cast<hipStream_t>(stream)), "pack launch");
}

ekv_status ekv_e4m3_to_f16(const uint8_t* codes, int32_t n, void* out, int32_t method, int32_t scale_exp,
                           void* stream) {
  if (n < 0) return fail(EKV_ERR_INVALID_ARG, "n %d < 0", n);
  if (method < 0 || method > 1) return fail(EKV_ERR_INVALID_ARG, "method must be 0 or 1");
  if (scale_exp < -126 || scale_exp > 127) return fail(EKV_ERR_INVALID_ARG, "scale_exp %d outside -126..127", scale_exp);
  if (n == 0) return ok();
  if (!codes || !out) return fail(EKV_ERR_INVALID_ARG, "codes and out are required");
  return hip_status(ekv::launch_e4m3_to_f16(codes, n, static_cast<uint16_t*>(out), method, scale_exp,
                                            static_cast<hipStream_t>(stream)),
                    "e4m3 launch");
}

}  // extern "C"

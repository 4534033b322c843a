/*
 * ekv.h — C ABI of libekv.so: attention over a mixed-fidelity paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (page titles as published):
 *   [ekv]  "Does Execution Require Target KV Fidelity? A Mixed-Fidelity KV
 *          Runtime for LLM Serving" (ElasticKV).
 *   [asym] "Memory-Traffic Saturation in Autoregressive Transformer Decode"
 *          (asymmetric K16/V8 KV cache).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, densely packed in the layouts stated below.  The library never
 *     allocates, frees or synchronizes; every launch is asynchronous on
 *     `stream` (a hipStream_t; NULL = the default stream).
 *   - Page layout (NHD): a page holds EKV_PAGE_SIZE tokens, each token all
 *     KV heads, each head `head_dim` contiguous elements:
 *     pool[page][slot][kv_head][d].  [asym] "What changes in vLLM's prefill
 *     routing?": NHD layout, page size 16, FP16 keys, FP8 E4M3 values.
 *   - FP8 values use the OCP E4M3FN encoding (bias 7, max 448, NaN 0x7F/0xFF).
 *   - Grouped-query attention: query head h reads KV head
 *     h / (num_q_heads / num_kv_heads).
 *   - Supported shapes: head_dim 64 or 128; num_q_heads / num_kv_heads in
 *     {1, 2, 4, 8}; page_size 16.  Others return EKV_ERR_UNSUPPORTED.
 *   - Errors: arguments are checked on the host before any launch; a non-OK
 *     status means nothing was launched.  ekv_last_error() then returns a
 *     thread-local message.  Launch failures return EKV_ERR_HIP.  No C++
 *     exception crosses the ABI.
 *   - Device-resident contents (page ids, flags, lengths, offsets) cannot be
 *     checked on the host.  Kernels bound-check them before any memory
 *     access: an out-of-range page id, an unknown fidelity flag, or prompt
 *     offsets outside the buffers never cause an out-of-bounds access; the
 *     affected output rows are written as NaN instead.
 *   - Output slices: each call writes only its own rows; pass an offset
 *     pointer to write a slice of a larger batch tensor ([asym] figure
 *     "Fresh prefill gets a fast path inside a mixed batch": each path writes
 *     its own output slice in the original request order).
 */
#ifndef EKV_H_
#define EKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EKV_ABI_VERSION 1
#define EKV_PAGE_SIZE 16
#define EKV_FIDELITY_TARGET 0   /* FP16 K + FP16 V                        */
#define EKV_FIDELITY_COMPACT 1  /* FP16 K + E4M3 V + fp32 scale/page/head  */
#define EKV_FIDELITY_BASE 2     /* ElasticKV BASE: high FP16 byte of K and V,
                                   two pages per TARGET block (elastic decode) */
#define EKV_MAX_PREFILL_TOKENS 8192 /* [asym] route rule: prompts of at most 8,192 tokens */
#define EKV_DECODE_BALANCED (-1)    /* decode plan: equal shares of all page-heads per workgroup */
#define EKV_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20) /* static scratch of the allocation-free decode */

typedef enum {
  EKV_OK = 0,
  EKV_ERR_INVALID_ARG = 1,         /* null pointer, bad size or stride      */
  EKV_ERR_UNSUPPORTED = 2,         /* shape outside the supported set       */
  EKV_ERR_WORKSPACE_TOO_SMALL = 3, /* gather larger than the workspace      */
  EKV_ERR_NOT_ELIGIBLE = 4,        /* prompt outside the prefill route rule */
  EKV_ERR_HIP = 5                  /* a HIP launch failed                   */
} ekv_status;

typedef enum { EKV_F16 = 0, EKV_F32 = 1 } ekv_dtype;

/*
 * The paged KV of one attention layer: two physical pools.
 * [ekv] section 3.2 and appendix B.3: a TARGET page and a compact page share
 * one attention output interface; a per-page mode selects the load path.
 * [asym] "What changes in vLLM's prefill routing?": compact pages keep FP16
 * keys and store values as E4M3 with value scales.
 *
 *   k_target, v_target : fp16 [n_target_pages][16][num_kv_heads][head_dim]
 *   k_compact          : fp16 [n_compact_pages][16][num_kv_heads][head_dim]
 *   v_compact          : u8 E4M3FN [n_compact_pages][16][num_kv_heads][head_dim]
 *   v_scale            : fp32 [n_compact_pages][num_kv_heads]; the value of a
 *                        compact element is e4m3(byte) * v_scale[page][head]
 * A pool that is not used may be NULL with its page count 0.  Page counts
 * must be below 2^28.  Scales must be positive normal fp32 values.
 *
 * ElasticKV BASE pages ([ekv] section 3.1, figure 3(b)) live in the TARGET
 * pools: BASE page id b is half (b & 1) of TARGET block b >> 1, i.e. the
 * block's first or second 16 x num_kv_heads x head_dim bytes, laid out
 * [slot][kv_head][d]; each byte is the high byte of an FP16 value.
 */
typedef struct {
  const void* k_target;
  const void* v_target;
  int32_t n_target_pages;
  const void* k_compact;
  const uint8_t* v_compact;
  const float* v_scale;
  int32_t n_compact_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size; /* must be EKV_PAGE_SIZE */
} ekv_paged_kv;

/* Version of this ABI (EKV_ABI_VERSION). */
int32_t ekv_abi_version(void);

/* Identity of the sources this library was built from: the sha256 (hex) of
 * the code of the .hip and .hpp kernel sources and of this header (comments
 * and whitespace removed), taken by the build script. */
const char* ekv_build_id(void);

/* Static description of a status code. */
const char* ekv_status_string(ekv_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* ekv_last_error(void);

/*
 * Decode split plan: how many pages one split of a sequence covers when
 * `pages_per_split` is 0 (automatic).  Pure host function.
 */
int32_t ekv_decode_pages_per_split(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len);

/*
 * Decode split plan from HOST-side sequence lengths (int32 [batch], host
 * memory), for callers whose scheduler knows them: batches of near-equal
 * lengths get one balanced round (one split per sequence and KV head when
 * there are 192..256 or at least 512 such groups, else about 512 split
 * workgroups), except where that plan would launch between one and two
 * rounds of split workgroups (more than 768, at most 1,536), which get
 * EKV_DECODE_BALANCED; ragged batches (up to 2,048 sequences) get
 * EKV_DECODE_BALANCED, larger ragged ones small splits.  Pass the result as
 * `pages_per_split`.  Pure host function; NULL or empty input returns 16.
 */
int32_t ekv_decode_plan_pages_per_split(const int32_t* seq_lens_host, int32_t batch,
                                        int32_t num_kv_heads);

/*
 * Scratch bytes ekv_decode_attention needs for these sizes (split-K partial
 * results).  `pages_per_split` 0 = the automatic plan.  0 when the plan has
 * a single split per sequence: the output is then written without partials
 * and scratch may be NULL.  Pure host function.
 */
size_t ekv_decode_scratch_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_seq_len, int32_t pages_per_split);

/*
 * GQA decode attention: one query token per sequence over its paged KV, in
 * one launch for any mix of TARGET and compact pages.
 * [asym] "What changes in vLLM's prefill routing?": decode reads persistent
 * FP16 keys and FP8 values, and value scales apply in attention.
 * [ekv] section 3.2: TARGET and compact pages execute in one batch and share
 * one output interface; compact values are expanded in registers, never
 * materialized as TARGET.
 *
 *   q          fp16 [batch][num_q_heads][head_dim]
 *   page_table int32 [batch][pt_stride]: physical page of logical page j of
 *              sequence b (token t lives in page t/16, slot t%16); ids index
 *              the pool that the page's flag selects.
 *   fidelity   u8 [batch][pt_stride]: EKV_FIDELITY_TARGET or _COMPACT.  May
 *              be NULL when exactly one pool is given: every page then uses
 *              that pool.
 *   seq_lens   int32 [batch]: tokens of each sequence, including the token
 *              being decoded (its K/V is already in the cache); the query
 *              attends to tokens [0, len).  Values are clamped to
 *              [0, max_seq_len]; len 0 gives out = 0 and lse = -inf.
 *   max_seq_len  host upper bound of seq_lens (sizes the launch);
 *              pt_stride must be >= ceil(max_seq_len / 16).
 *   sm_scale   softmax scale (typically 1/sqrt(head_dim)).
 *   out        [batch][num_q_heads][head_dim] in `out_dtype`.  In EKV_F16 the
 *              value is the round-to-nearest-even of the EKV_F32 result.
 *   lse        optional fp32 [batch][num_q_heads]: natural-log normalizer
 *              max_t s_t + ln sum_t exp(s_t - max_t s_t).
 *   pages_per_split  split-K granularity (0 = automatic; else 1..512), or
 *              EKV_DECODE_BALANCED (batch <= 2,048): all page-heads of the
 *              batch, ordered (sequence, KV head, page), are cut into equal
 *              contiguous ranges, one per workgroup, in whole rounds of one
 *              workgroup per CU (more rounds only to keep each range within
 *              512 pages); a sequence that one range holds whole is written
 *              directly, the pieces of a cut one are merged by a second
 *              kernel.  Evens out ragged lengths.  Split plans with more
 *              than one split per sequence also end with the merge kernel.
 *   scratch    device buffer of at least ekv_decode_scratch_bytes(...) bytes
 *              (same arguments), 256-byte aligned; contents are overwritten
 *              and need no initial value.  Unused (may be NULL) when that
 *              size is 0.  Calls that overlap in time must not share a
 *              scratch buffer.
 * Sequences that reference an out-of-range page id or an unknown flag get
 * NaN outputs and NaN lse.
 */
ekv_status ekv_decode_attention(const ekv_paged_kv* kv, const void* q, int32_t batch,
                                int32_t num_q_heads, const int32_t* page_table, int32_t pt_stride,
                                const uint8_t* fidelity, const int32_t* seq_lens,
                                int32_t max_seq_len, float sm_scale, void* out, ekv_dtype out_dtype,
                                float* lse, int32_t pages_per_split, void* scratch,
                                size_t scratch_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): ekv_decode_attention with the same arguments except scratch,
 * whose role is taken by a fixed device array inside the library of
 * EKV_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held until the process ends.
 * Same plans, kernels and results as ekv_decode_attention (bit for bit).
 *
 *   A plan whose ekv_decode_scratch_bytes(...) exceeds 8 MiB returns
 *   EKV_ERR_WORKSPACE_TOO_SMALL before any launch (the balanced plan needs
 *   about 4.2 KB per workgroup at 4 query heads per KV head and head dim
 *   128, so it fits 1,792 workgroups, i.e. 7 rounds; the split plan needs
 *   batch x num_q_heads x splits x (head_dim + 2) x 4 bytes).
 *   The call allocates and frees nothing.  The first call on a device looks
 *   up that device's copy of the array (once); it launches on the stream's
 *   device (the current device for a NULL stream).  Nothing in the array has
 *   to start at zero: every partial result is written before it is read.
 *   Calls share the array of their GPU: two calls that overlap in time on
 *   one GPU (other streams, or other host threads without ordering) race.
 */
ekv_status ekv_decode_attention_noalloc(const ekv_paged_kv* kv, const void* q, int32_t batch,
                                        int32_t num_q_heads, const int32_t* page_table, int32_t pt_stride,
                                        const uint8_t* fidelity, const int32_t* seq_lens, int32_t max_seq_len,
                                        float sm_scale, void* out, ekv_dtype out_dtype, float* lse,
                                        int32_t pages_per_split, void* stream);

/*
 * Elastic decode: ekv_decode_attention over pages that may also be ElasticKV
 * BASE pages.  [ekv] section 3.2 and appendix B.3: a batch-level BASE
 * indicator lets batches without BASE skip the elastic machinery; batches
 * with BASE carry either a per-page mode table (general path) or per-sequence
 * boundaries of the common TARGET-BASE-TARGET layout (structured path); a
 * BASE value is its stored byte in the high position with a zero low byte,
 * read in registers, with no scale.
 *
 *   has_base     0: exactly ekv_decode_attention (flags 0/1; base_bounds NULL).
 *                1: the batch may hold BASE pages; then give exactly one of
 *   fidelity     u8 [batch][pt_stride] with values 0, 1 or 2 (EKV_FIDELITY_*),
 *   base_bounds  int32 [batch][2] (device): logical pages [lo, hi) of
 *                sequence b are BASE, all others TARGET (no flag table).
 * Other arguments, scratch sizing and the NaN rule for bad ids or flags are
 * those of ekv_decode_attention.  has_base = 1 needs a non-empty TARGET pool.
 */
ekv_status ekv_decode_attention_elastic(const ekv_paged_kv* kv, const void* q, int32_t batch,
                                        int32_t num_q_heads, const int32_t* page_table,
                                        int32_t pt_stride, const uint8_t* fidelity,
                                        const int32_t* base_bounds, int32_t has_base,
                                        const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                        void* out, ekv_dtype out_dtype, float* lse,
                                        int32_t pages_per_split, void* scratch, size_t scratch_bytes,
                                        void* stream);

/*
 * Compact-prefill gather: copy the listed compact pages into a bounded FP16
 * workspace.  [asym] "What changes in vLLM's prefill routing?" (figure "Fresh
 * prefill gets a fast path inside a mixed batch"): stored K16/V8 pages are
 * gathered into one shared FP16 payload of at most 4,096 pages and V8 is cast
 * to FP16.
 *
 *   page_ids   int32 [n_pages], indices into the compact pool.
 *   ws_k, ws_v fp16 [ws_capacity_pages][16][num_kv_heads][head_dim]; page i of
 *              the workspace receives pool page page_ids[i], so the workspace
 *              is token-major [n_pages*16][num_kv_heads][head_dim].
 *   apply_scale 0: ws_v = fp16(e4m3(byte))            (exact cast)
 *               1: ws_v = fp16(fp32(e4m3(byte)) * fp32(scale))  (one fp32
 *                  multiply, round-to-nearest-even, then one fp16 rounding,
 *                  round-to-nearest-even)
 *   Keys are copied bit for bit.  E4M3 NaN codes become FP16 NaN.
 * n_pages > ws_capacity_pages returns EKV_ERR_WORKSPACE_TOO_SMALL.  An
 * out-of-range page id fills that workspace page with NaN.
 */
ekv_status ekv_gather_compact_pages(const ekv_paged_kv* kv, const int32_t* page_ids,
                                    int32_t n_pages, int32_t apply_scale, void* ws_k, void* ws_v,
                                    int32_t ws_capacity_pages, void* stream);

/*
 * Causal FP16 prefill attention of fresh prompts over contiguous K/V rows
 * (the gather workspace).  [asym] "What changes in vLLM's prefill routing?":
 * whole fresh prompts with no cached prefix, FP16 Q/K/V, causal attention
 * without sliding windows, attention sinks or soft caps.
 *
 *   q            fp16 [q_rows][num_q_heads][head_dim]; prompt p owns rows
 *                [cu_seqlens_q[p], cu_seqlens_q[p+1]).
 *   k, v         fp16 [kv_rows][num_kv_heads][head_dim]; prompt p's keys are
 *                rows [kv_start[p], kv_start[p] + len_p), len_p = its query
 *                count (q_len == kv_len).
 *   cu_seqlens_q int32 [n_prompts + 1], kv_start int32 [n_prompts] (device).
 *   max_len      host bound of every len_p; > EKV_MAX_PREFILL_TOKENS returns
 *                EKV_ERR_NOT_ELIGIBLE (the caller chunks or falls back).
 *   causal       1: query i sees keys 0..i of its prompt; 0: all len_p keys.
 *   sm_scale     softmax scale; must be finite and > 0 (EKV_ERR_INVALID_ARG
 *                otherwise: a row's max is taken before scaling).
 *   out          [q_rows][num_q_heads][head_dim] in out_dtype (F16 = RNE of
 *                the F32 result); rows outside every prompt are not written.
 *   lse          optional fp32 [q_rows][num_q_heads], natural log.
 * A prompt whose offsets leave the buffers or exceed max_len is not read;
 * its in-bounds output rows are written as NaN.
 */
ekv_status ekv_prefill_attention(const void* q, int32_t q_rows, const void* k, const void* v,
                                 int32_t kv_rows, const int32_t* cu_seqlens_q,
                                 const int32_t* kv_start, int32_t n_prompts, int32_t max_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t causal, float sm_scale, void* out, ekv_dtype out_dtype,
                                 float* lse, void* stream);

/*
 * Direct paged prefill: causal FP16 prefill of fresh prompts that reads each
 * prompt's own pages (no workspace).  [asym] "Existing fallback: mixed-type
 * prefill" (a prefill kernel on stored K16/V8 pages) and "What changes in
 * vLLM's prefill routing?" (the gather route this replaces); [ekv] section
 * 3.2 (TARGET and compact pages read in one launch).
 *
 *   q            fp16 [q_rows][num_q_heads][head_dim]; prompt p owns rows
 *                [cu_seqlens_q[p], cu_seqlens_q[p+1]) (device int32 [n+1]).
 *   page_table   int32 [n_prompts][pt_stride] (device): token t of prompt p
 *                is in page page_table[p][t/16], slot t%16; q_len == kv_len.
 *   fidelity     u8 [n_prompts][pt_stride] or NULL when exactly one pool is
 *                given (as in ekv_decode_attention).
 *   max_len      host bound of every prompt length; > EKV_MAX_PREFILL_TOKENS
 *                returns EKV_ERR_NOT_ELIGIBLE; pt_stride >= ceil(max_len/16).
 *   causal, sm_scale, out, out_dtype, lse: as in ekv_prefill_attention.
 * Values: a TARGET page's FP16 V as stored; a compact page's V as
 * fp16(fp32(e4m3) * fp32(scale)) — the scaled gather's values, so the result
 * equals gather + ekv_prefill_attention bit for bit.  A page with an
 * out-of-pool id or an unknown flag poisons its prompt from the start of
 * the 64-token key tile that holds it: those rows (every causal row that
 * attends to the page among them) are written as NaN, and so may be up to
 * 255 rows before it (the rows sharing a workgroup with them); earlier
 * rows are computed.  Without the causal mask the whole prompt is NaN.  An
 * over-long prompt (len > max_len) is written as NaN.
 */
ekv_status ekv_prefill_paged_attention(const ekv_paged_kv* kv, const void* q, int32_t q_rows,
                                       const int32_t* cu_seqlens_q, const int32_t* page_table,
                                       int32_t pt_stride, const uint8_t* fidelity, int32_t n_prompts,
                                       int32_t max_len, int32_t num_q_heads, int32_t causal,
                                       float sm_scale, void* out, ekv_dtype out_dtype, float* lse,
                                       void* stream);

/*
 * Cache writer, TARGET append: store new tokens' K and V rows into TARGET
 * pages.  [ekv] section 3.2 and appendix B.3: newly appended KV is kept at
 * target fidelity in the protected recent window.
 *
 *   kv           the layer's pools; this call WRITES through kv->k_target and
 *                kv->v_target (writable device memory; n_target_pages * 16
 *                must be below 2^31).
 *   k_new, v_new fp16 [n_tokens][num_kv_heads][head_dim] (device).
 *   slot_mapping int32 [n_tokens] (device): token t goes to TARGET page
 *                slot_mapping[t] / 16, slot slot_mapping[t] % 16; all KV heads
 *                of the row are copied bit for bit.  A negative or
 *                out-of-pool slot skips that token.  Slots must be distinct
 *                (two tokens on one slot race).
 */
ekv_status ekv_append_tokens(const ekv_paged_kv* kv, const void* k_new, const void* v_new,
                             const int32_t* slot_mapping, int32_t n_tokens, void* stream);

/*
 * Cache writer, page quantizer: write compact pages (K16 + E4M3 V + scale)
 * from FP16 token rows, with the scale finalized over the whole page.
 * [asym] "What changes in vLLM's prefill routing?" and the table "Historical
 * reported implementation checks": keys stay bit-exact, values become E4M3
 * with value scales.  [ekv] section 3.3: a TARGET -> compact transition
 * rewrites whole pages.  One call serves a demotion (source = the TARGET
 * pool seen as rows, row = page * 16) and a prompt's fresh rows.
 *
 *   kv             the layer's pools; this call WRITES through kv->k_compact,
 *                  kv->v_compact and kv->v_scale (writable device memory).
 *   k_src, v_src   fp16 [src_rows][num_kv_heads][head_dim] (device); must not
 *                  overlap the compact pool.
 *   src_row_start  int32 [n_pages]: page i is made of source rows
 *                  src_row_start[i] .. src_row_start[i] + n_valid[i] - 1.
 *   n_valid        int32 [n_pages] in 0..16, or NULL for 16 each.
 *   dst_pages      int32 [n_pages]: compact page ids written (distinct).
 * Per KV head h of page i, with absmax over the n_valid rows x head_dim:
 *   v_scale[dst][h] = absmax / 448 (fp32, round to nearest even), or 1.0
 *                     when absmax is 0;
 *   code = E4M3FN(fp32(v) / scale): correctly rounded fp32 quotient, then the
 *          nearest E4M3 value, ties to even, saturating at +-448, NaN -> 0x7F;
 *   K    = bit copy.  Slots past n_valid get K = +0.0 and code 0x00.
 * Source rows must hold finite values.  A page whose rows leave [0,
 * src_rows), whose n_valid is outside 0..16 or whose dst id is outside the
 * compact pool is skipped (nothing is written for it).
 */
ekv_status ekv_quantize_pages(const ekv_paged_kv* kv, const void* k_src, const void* v_src,
                              int64_t src_rows, const int32_t* src_row_start,
                              const int32_t* n_valid, const int32_t* dst_pages, int32_t n_pages,
                              void* stream);

/*
 * ElasticKV demotion pack: TARGET pairs -> BASE blocks.  [ekv] section 3.1
 * and appendix B.2: the GPU packs the high-order bytes of a pair's two TARGET
 * blocks into one block (the pair's BASE layout) and the other block is
 * returned to the allocator.
 *
 *   kv            WRITES through kv->k_target and kv->v_target.
 *   src_a, src_b  int32 [n_pairs] (device): the pair's TARGET blocks.
 *   dst           int32 [n_pairs] (device): the block that receives the pair;
 *                 half 0 = high bytes of src_a (BASE page 2 dst), half 1 =
 *                 high bytes of src_b (BASE page 2 dst + 1), for K and V.
 *                 dst may equal src_a or src_b (in place: both blocks are
 *                 read before it is written).  Blocks of different pairs
 *                 must not overlap.
 * A pair with an id outside the TARGET pool is skipped.  num_kv_heads *
 * head_dim above 2048 returns EKV_ERR_UNSUPPORTED.
 */
ekv_status ekv_pack_base_pairs(const ekv_paged_kv* kv, const int32_t* src_a, const int32_t* src_b,
                               const int32_t* dst, int32_t n_pairs, void* stream);

/*
 * Diagnostic for the device E4M3 decoding used by the kernels: out[i] =
 * fp16(e4m3(codes[i]) * 2^scale_exp), scale_exp in -126..127.  method 0 =
 * the decode kernel's conversion instruction (codes packed four per 32-bit
 * word, the instruction's power-of-two scale; the decode kernel hands it
 * only exponents in -15..7, where every result is exact); method 1 = the
 * gather's arithmetic (fp32 product rounded to nearest even, then fp16
 * rounded to nearest even).  codes u8 [n], out fp16 [n] (device).  Other
 * methods or exponents return EKV_ERR_INVALID_ARG.
 */
ekv_status ekv_e4m3_to_f16(const uint8_t* codes, int32_t n, void* out, int32_t method, int32_t scale_exp,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EKV_H_ */

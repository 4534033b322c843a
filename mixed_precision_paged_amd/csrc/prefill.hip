// Causal FP16 flash prefill over the contiguous gather workspace (MFMA).
//
// Source: "Memory-Traffic Saturation in Autoregressive Transformer Decode",
// section "What changes in vLLM's prefill routing?": whole fresh prompts with
// no cached prefix are prefilled with FP16 Q, K and V from the gathered
// workspace; causal attention without sliding window, sinks or soft cap.
// The CPU replay note on the same page names FP16 probability rounding as the
// expected difference from ideal arithmetic: P is rounded to fp16 for the
// P.V product, accumulation is fp32.
//
// This is a dense QK^T / PV contraction, so it runs on the matrix cores
// (v_mfma_f32_32x32x16_f16, gfx950).  Workgroup = NW blocks of 32 query
// rows of one prompt: 32 NW positions of one query head, or (head dim 128,
// 4 wavefronts) 32 positions of up to 4 query heads that share a KV head;
// each wavefront owns one block.  Per 32-key unit each wavefront computes
//     S^T[key][q] = K . Q^T      (A = K from LDS, B = Q in registers)
//     O^T[d][q]  += V^T . P^T    (A = V^T from LDS, B = P^T in registers)
// so that with the 32x32 output layout every per-query quantity (running max,
// sum, rescale factor) lives in the lane whose column is that query: lane l
// holds column l%32 and half of its rows; a single xor-32 exchange completes a
// column reduction.  The key order inside the P.V contraction follows the
// S^T register layout, and V^T is read in the same order.
// Launch order: workgroups are mapped so that each XCD (8 per MI355X, each
// with its own L2) walks a contiguous range of (prompt, KV head) groups, so
// the K/V rows the group's query heads share stay in one L2; within a group
// the longest (last) causal row tiles of all its query heads start first.
//
// Sources: the gather workspace, or the direct route over pages
// ("Memory-Traffic Saturation ...", section "Existing fallback: mixed-type
// prefill"; ElasticKV section 3.2): the prompt's own page-table row, TARGET
// pages as stored, compact pages' E4M3 values expanded while the tile is
// staged with the scaled gather's rounding (fp16(fp32(e4m3) * fp32(scale))),
// so both routes feed the MFMAs identical operands, and a row's arithmetic
// does not depend on the workgroup size: the two routes agree bit for bit.
//   prefill_pipe_kernel   head dim 128, both sources: K and V tiles go
//                         straight from memory into swizzled LDS by buffer
//                         loads; V^T operands come from transposing LDS
//                         reads; a three-stage pipeline over 32-key units
//                         (described at the kernel).  Paged: each wavefront
//                         stages one page (4 wavefronts) or half a page (8)
//                         of each 64-key tile through per-page
//                         descriptors; a compact page's codes land in a
//                         per-wavefront LDS area and are expanded into the V
//                         tile before the barrier that publishes it.
//                         Query rows (8 wavefronts) and fp16 output rows
//                         pass through LDS so that every load and store
//                         instruction moves whole 256-byte rows.
//   prefill_kernel        head dim 64, both sources: K and V staged through
//                         registers; V^T transposed with byte permutes on its
//                         way into padded LDS tiles; one 64-key tile per step.
#include <utility>

#include "ekv_device.hpp"
#include "ekv_internal.hpp"

namespace ekv {
namespace {

constexpr int kM = 128;        // query rows per workgroup
constexpr int kN = 64;         // keys per tile
constexpr int kThreads = 256;
constexpr float kTau = 8.0f;
constexpr float kOver = 256.0f;  // 2^kTau: a lane's weight sum of one unit that starts a rescale
constexpr float kNegBig = -1.0e30f;
constexpr int kXcds = 8;
constexpr int kMaxPromptPages = 512;  // paged source: prompts of at most 8192 tokens

template <int D>
struct SmemK {
  static constexpr int kStride = D + 8;    // K row stride (halves): 16 B pad
  f16 k[kN * kStride];
};
template <int D>
struct SmemV {
  static constexpr int vStride = kN + 4;   // V^T row stride (halves): 8 B pad
  f16 vt[D * vStride];
};

// V^T column swizzle of the paged source: the 8-byte key quad kq of V^T row
// d is stored at quad kq ^ ((d / 32) & 3).  There a wavefront stages the key
// quads of its pages for every d-octet, and the plain layout would put those
// stores on a fraction of the LDS banks; the swizzle spreads them and keeps
// the MFMA reads conflict-free.  The workspace source stages sixteen
// key quads per wavefront and is faster unswizzled.  The value depends on d / 8
// only: one per staging thread (rows 8 oc .. 8 oc + 7) and per MFMA read.
template <bool SWZ>
__device__ __forceinline__ int vt_swz(int d) {
  return SWZ ? (d >> 5) & 3 : 0;
}

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <int D>
struct KRegs {
  static constexpr int KCH = kN * D / 8 / kThreads;  // 16-byte K chunks per thread
  uint4 k[KCH];
};
struct VRegs {
  uint2 vlo[4];  // 4 key rows x 8 d of one (key quad, d octet) unit: d 0..3 of
  uint2 vhi[4];  // each row in vlo, d 4..7 in vhi; for a compact page (paged
                 // source) vlo holds the row's 8 E4M3 codes and vhi is unused
  float vscale;
  bool v_codes;
};

// fp32 -> fp16 pair, round to nearest even each.
__device__ __forceinline__ uint32_t pack_rne(float a, float b) {
  f16x2 r;
  r.x = (f16)a;
  r.y = (f16)b;
  return bits(r);
}

// Eight E4M3 codes -> eight fp16 values fp16(fp32(code) * s): the code is
// exact in fp32, one fp32 multiply (round to nearest even), one fp16 rounding.
__device__ __forceinline__ uint4 expand8(uint2 w, float s) {
#pragma clang fp contract(off)
  const f32x2 a = e4m3x2_f32(w.x, false), b = e4m3x2_f32(w.x, true);
  const f32x2 c = e4m3x2_f32(w.y, false), d = e4m3x2_f32(w.y, true);
  return make_uint4(pack_rne(a.x * s, a.y * s), pack_rne(b.x * s, b.y * s),
                    pack_rne(c.x * s, c.y * s), pack_rne(d.x * s, d.y * s));
}

// Tile loads are buffer loads through per-prompt descriptors (SGPRs) whose
// range ends at the prompt's last key row of this KV head, so rows past the
// prompt read as zeros (no per-load branch).  Per-lane byte offsets are fixed
// for the whole loop; the tile's first row goes in the scalar offset.
template <int D>
__device__ __forceinline__ void load_k(KRegs<D>& r, __amdgpu_buffer_rsrc_t kr, const uint32_t* koff,
                                       uint32_t tile_off) {
#pragma unroll
  for (int i = 0; i < KRegs<D>::KCH; ++i) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[i], tile_off, 0);
    r.k[i] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

__device__ __forceinline__ void load_v(VRegs& r, __amdgpu_buffer_rsrc_t vr, const uint32_t* voff,
                                       uint32_t tile_off) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[i], tile_off, 0);
    r.vlo[i] = make_uint2(x.x, x.y);
    r.vhi[i] = make_uint2(x.z, x.w);
  }
  r.v_codes = false;
}

// Writes a staged K tile to LDS, row-major.
template <int D>
__device__ __forceinline__ void store_k(SmemK<D>& s, const KRegs<D>& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < KRegs<D>::KCH; ++i) {
    const int idx = t + kThreads * i;
    const int key = idx / (D / 8), ch = idx % (D / 8);
    *reinterpret_cast<uint4*>(&s.k[key * SmemK<D>::kStride + 8 * ch]) = r.k[i];
  }
}

// Writes a staged V tile to LDS transposed.  The V unit (key quad kq, d octet
// oc) of this thread holds keys 4kq..4kq+3, d 8oc..8oc+7.
template <int D, bool SWZ>
__device__ __forceinline__ void store_v(SmemV<D>& s, const VRegs& r, int kq, int oc, bool v_active,
                                        int valid_keys) {
  if (v_active) {
    uint4 v[4];
    // the two half-wavefronts may hold different pages (a select)
    const bool codes = r.v_codes;
    if (codes) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = expand8(r.vlo[i], r.vscale);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = make_uint4(r.vlo[i].x, r.vlo[i].y, r.vhi[i].x, r.vhi[i].y);
    }
    if (valid_keys < kN) {  // last tile of a prompt: value rows past its end are zero
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * kq + i >= valid_keys) v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    const uint32_t r0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
    const uint32_t r1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
    const uint32_t r2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
    const uint32_t r3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // d = 8*oc + 2w and 2w+1: four keys' values, key order 4kq..4kq+3
      const uint2 even = make_uint2(perm(r1[w], r0[w], 0x05040100u), perm(r3[w], r2[w], 0x05040100u));
      const uint2 odd = make_uint2(perm(r1[w], r0[w], 0x07060302u), perm(r3[w], r2[w], 0x07060302u));
      const int d = 8 * oc + 2 * w;
      const int kqs = kq ^ vt_swz<SWZ>(8 * oc);
      *reinterpret_cast<uint2*>(&s.vt[d * SmemV<D>::vStride + 4 * kqs]) = even;
      *reinterpret_cast<uint2*>(&s.vt[(d + 1) * SmemV<D>::vStride + 4 * kqs]) = odd;
    }
  }
}

// Paged source: per-workgroup pool bases (already offset to KV head g) and row sizes.
struct PagedSrc {
  const char* kt;
  const char* vt;
  const char* kc;
  const char* vc;
  uint32_t rowb;     // bytes per fp16 token row (all KV heads)
  uint32_t rowb8;    // bytes per E4M3 token row
  uint32_t range16;  // descriptor range of one head's fp16 page: 15 rows + D halves
  uint32_t range8;   // the same for an E4M3 page
};

// Metadata of the 4 pages of one tile: meta = (phys << 1) | kind, or < 0 for
// a page past the prompt; the scale of a compact page.  Read from LDS one
// tile ahead of its use (two 16-byte reads) and made wave-uniform only where
// it is used, so the LDS latency never stalls the load issue.
struct TileMetaRaw {
  int4 m;
  float4 s;
};
struct TileMeta {
  int m[4];
  float s[4];
};

__device__ __forceinline__ TileMetaRaw read_tile_meta(const int* s_meta, const float* s_scale, int it) {
  return TileMetaRaw{*reinterpret_cast<const int4*>(s_meta + 4 * it),
                     *reinterpret_cast<const float4*>(s_scale + 4 * it)};
}

__device__ __forceinline__ float rfl(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ TileMeta uniform_meta(const TileMetaRaw& r) {
  TileMeta t;
  t.m[0] = __builtin_amdgcn_readfirstlane(r.m.x);
  t.m[1] = __builtin_amdgcn_readfirstlane(r.m.y);
  t.m[2] = __builtin_amdgcn_readfirstlane(r.m.z);
  t.m[3] = __builtin_amdgcn_readfirstlane(r.m.w);
  t.s[0] = rfl(r.s.x);
  t.s[1] = rfl(r.s.y);
  t.s[2] = rfl(r.s.z);
  t.s[3] = rfl(r.s.w);
  return t;
}

// Descriptors of one page (meta = (phys << 1) | kind, always a valid page:
// pages past the prompt were staged as a copy of its page 0).  Each range is
// one head's page; rows past the prompt end are masked (K) or zeroed (V) in
// the tile instead.  V keeps its base and the code flag: the loads build the
// descriptors of its two row halves.
struct PageDesc {
  __amdgpu_buffer_rsrc_t k;
  const char* vbase;
  float scale;
  bool codes;
};

__device__ __forceinline__ PageDesc page_desc(PagedSrc src, int meta, float scale) {
  PageDesc pd;
  const int64_t phys = meta >> 1;
  pd.codes = meta & 1;
  const int64_t off16 = phys * kPage * src.rowb;
  pd.k = __builtin_amdgcn_make_buffer_rsrc((void*)((pd.codes ? src.kc : src.kt) + off16), (short)0,
                                           src.range16, kBufferFlags);
  pd.vbase = pd.codes ? src.vc + phys * kPage * src.rowb8 : src.vt + off16;
  pd.scale = scale;
  return pd;
}

// V rows 4(kq%4) .. +3 of one page for this thread's unit, each as two 8-byte
// halves.  The same eight loads serve both kinds, so both write the same
// registers and no wait or spill follows from the kind: an fp16 page gives
// d 0..3 and d 4..7; a compact page gives its 8 codes in the low half while
// the high half reads through a zero-range descriptor (no memory access).
__device__ __forceinline__ void load_v_page(uint2* lo, uint2* hi, const PageDesc& pd, const PagedSrc& src,
                                            uint32_t voff16, uint32_t voff8) {
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)pd.vbase, (short)0, pd.codes ? src.range8 : src.range16, kBufferFlags);
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)pd.vbase, (short)0, pd.codes ? 0u : src.range16, kBufferFlags);
  const uint32_t off = pd.codes ? voff8 : voff16;
  const uint32_t stride = pd.codes ? src.rowb8 : src.rowb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(vr, off, i * stride, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(hr, voff16 + 8u, i * src.rowb, 0);
    lo[i] = make_uint2(a.x, a.y);
    hi[i] = make_uint2(b.x, b.y);
  }
}

// Paged loads of tile t (keys 64 t .. 64 t + 63 = prompt pages 4 t .. 4 t + 3),
// head dim 64.  K chunk i of this thread lies in tile page 2 i + wave / 2; the
// V unit's page is that of its half-wavefront.
template <int D>
__device__ __forceinline__ void load_k_paged(KRegs<D>& r, PagedSrc src, const TileMetaRaw& raw, int wave,
                                             uint32_t koff) {
  const TileMeta tm = uniform_meta(raw);
  const bool hi = wave >> 1;
#pragma unroll
  for (int i = 0; i < KRegs<D>::KCH; ++i) {
    const PageDesc pd = page_desc(src, hi ? tm.m[2 * i + 1] : tm.m[2 * i], hi ? tm.s[2 * i + 1] : tm.s[2 * i]);
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(pd.k, koff, 0, 0);
    r.k[i] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

template <int D>
__device__ __forceinline__ void load_v_paged(VRegs& r, PagedSrc src, const TileMetaRaw& raw, int wave, int lane,
                                             uint32_t voff16, uint32_t voff8) {
  const TileMeta tm = uniform_meta(raw);
  if (wave < 2) {  // 128 V units, two pages per wavefront
    const bool w1 = wave == 1;
    const PageDesc pa = page_desc(src, w1 ? tm.m[2] : tm.m[0], w1 ? tm.s[2] : tm.s[0]);
    const PageDesc pb = page_desc(src, w1 ? tm.m[3] : tm.m[1], w1 ? tm.s[3] : tm.s[1]);
    if (lane < 32) {
      load_v_page(r.vlo, r.vhi, pa, src, voff16, voff8);
      r.v_codes = pa.codes;
      r.vscale = pa.scale;
    } else {
      load_v_page(r.vlo, r.vhi, pb, src, voff16, voff8);
      r.v_codes = pb.codes;
      r.vscale = pb.scale;
    }
  }
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes bytes
// [16 l, 16 l + 16) after `dst` (wave-uniform); out-of-range lanes write zeros.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, f16* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

// Writes NaN to output rows [r_lo, r_hi) of head h (and their LSE).
template <int D>
__device__ void write_nan_rows(const PrefillParams& p, int64_t q0, int r_lo, int r_hi, int h) {
  const float qnan = __builtin_nanf("");
  const int64_t hq_row = (int64_t)p.num_q_heads * D;
  for (int64_t i = threadIdx.x; i < (int64_t)(r_hi - r_lo) * D; i += blockDim.x) {
    const int64_t rr = r_lo + i / D;
    const int64_t o = (q0 + rr) * hq_row + (int64_t)h * D + i % D;
    if (p.out_f32) static_cast<float*>(p.out)[o] = qnan;
    else static_cast<f16*>(p.out)[o] = (f16)qnan;
    if (p.lse && i % D == 0) p.lse[(q0 + rr) * p.num_q_heads + h] = qnan;
  }
}

// Work item of this workgroup: (prompt, query head, row tile).  Each XCD (own
// L2) takes a contiguous range of items, and within it the items are grouped
// by (prompt, KV head): the G query heads that read the same K/V rows run
// together.  Inside a group the row tiles go longest first across all G
// heads (a causal row tile's work grows with its index), so the long tiles
// start first and the short ones fill the end; ordering only within each
// head leaves a sawtooth of long tiles late in the range (about a fifth
// longer runs for 2048-token prompts in a list-schedule model).
struct WorkItem {
  int prompt, h, mt;
};
// Heads per workgroup of the head-dim-128 kernel.  At 4 wavefronts: the
// largest power of two dividing both the GQA group size G and 4, so that
// the wavefronts take HW query heads of one KV head times 4 / HW blocks of
// 32 positions and every wavefront of a causal workgroup ends within one
// 32-key unit of the others (one head per workgroup spreads them over 4
// units, and the early ones idle while the last ones finish): 3.0-3.6%
// faster on 512-1,500-token prompts.  At 8 wavefronts one head of 256
// positions measured as fast or faster on prompts of whole 256-row tiles
// (4 x 2048 1.9%, the paged source 1-3%), so those keep it.
__host__ __device__ __forceinline__ int heads_per_workgroup(int G, int NW) {
  if (NW != 4) return 1;
  const int low = G & -G;
  return low < NW ? low : NW;
}
// (prompt, first query head, row tile) of a workgroup of HW heads; the
// order is that of work_item, over groups of HW heads instead of heads.
__device__ __forceinline__ WorkItem work_item_heads(const PrefillParams& p, int n_mtiles, int HW) {
  const int total = (int)gridDim.x;
  const int bid = blockIdx.x;
  const int work = (total % kXcds == 0) ? (bid % kXcds) * (total / kXcds) + bid / kXcds : bid;
  const int GW = p.num_q_heads / p.num_kv_heads / HW;  // head groups per KV head
  const int per_group = GW * n_mtiles;
  const int grp = work / per_group, r = work % per_group;
  WorkItem wi;
  wi.mt = n_mtiles - 1 - r / GW;
  wi.h = ((grp % p.num_kv_heads) * GW + r % GW) * HW;
  wi.prompt = grp / p.num_kv_heads;
  return wi;
}
__device__ __forceinline__ WorkItem work_item(const PrefillParams& p, int n_mtiles) {
  const int total = (int)gridDim.x;
  const int bid = blockIdx.x;
  const int work = (total % kXcds == 0) ? (bid % kXcds) * (total / kXcds) + bid / kXcds : bid;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int per_group = G * n_mtiles;
  const int grp = work / per_group, r = work % per_group;
  WorkItem wi;
  wi.mt = n_mtiles - 1 - r / G;
  wi.h = (grp % p.num_kv_heads) * G + r % G;
  wi.prompt = grp / p.num_kv_heads;
  return wi;
}

// Paged source: stages the prompt's page ids, kinds and scales of pages
// 0 .. n_pages - 1 in LDS (meta = (phys << 1) | kind; scale 1 for a TARGET
// page).  Pages past the prompt get a copy of page 0, which is in bounds:
// their keys are masked and their values zeroed in the tile.  Returns false
// (the same on every thread) if a page id lies outside its pool or a flag is
// unknown; the caller then writes its rows as NaN.
__device__ bool stage_page_meta(const PrefillParams& p, int prompt, int g, int L, int n_pages, int* s_meta,
                                float* s_scale, int* s_bad) {
  if (threadIdx.x == 0) *s_bad = 0;
  __syncthreads();
  const int64_t pt_row = (int64_t)prompt * p.pt_stride;
  for (int j = threadIdx.x; j < n_pages; j += blockDim.x) {
    int meta = -2;
    float sc = 1.0f;
    if (kPage * j < L) {
      const int id = p.page_table[pt_row + j];
      const int kind = p.fidelity ? (int)p.fidelity[pt_row + j] : p.uniform_kind;
      const int n_pool = kind == 1 ? p.n_compact : p.n_target;
      if ((kind == 0 || kind == 1) && id >= 0 && id < n_pool) {
        meta = (id << 1) | kind;
        if (kind == 1) sc = p.v_scale[(int64_t)id * p.num_kv_heads + g];
      } else {
        *s_bad = 1;
      }
    }
    s_meta[j] = meta;
    s_scale[j] = sc;
  }
  __syncthreads();
  if (*s_bad) return false;
  for (int j = threadIdx.x; j < n_pages; j += blockDim.x)
    if (kPage * j >= L) {
      s_meta[j] = s_meta[0];
      s_scale[j] = s_scale[0];
    }
  __syncthreads();
  return true;
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p, int n_mtiles) {
  static_assert(D == 64, "head dim 128 runs prefill_pipe_kernel");
  constexpr int KS = D / 16;  // k-steps of 16 over the head dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  // K of tiles i + 1 (computing S ahead) and i + 2 (being stored), V of
  // tiles i (P.V) and i + 1 (being stored)
  __shared__ SmemK<D> kbuf[2];
  __shared__ SmemV<D> vbuf[2];
  // paged source: the prompt's page metadata for the tiles this workgroup reads
  __shared__ __attribute__((aligned(16))) int s_meta[PAGED ? kMaxPromptPages : 4];
  __shared__ __attribute__((aligned(16))) float s_scale[PAGED ? kMaxPromptPages : 4];
  __shared__ int s_bad;

  // XCD-aware work mapping (see header).
  const WorkItem wi = work_item(p, n_mtiles);
  const int prompt = wi.prompt, h = wi.h, mt = wi.mt;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = h / G;

  const int q0 = p.cu_seqlens_q[prompt];
  const int q1 = p.cu_seqlens_q[prompt + 1];
  if (q0 < 0 || q1 < q0 || q1 > p.q_rows) return;  // rows not addressable: nothing to write
  const int L = q1 - q0;
  const int m0 = mt * kM;
  const int kv0 = PAGED ? 0 : p.kv_start[prompt];
  const bool ok = PAGED ? (L <= p.max_len && L <= kMaxPromptPages * kPage &&
                           (int64_t)L <= (int64_t)p.pt_stride * kPage)
                        : (L <= p.max_len && kv0 >= 0 && (int64_t)kv0 + L <= p.kv_rows);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int r0 = m0 + 32 * wave;     // first row (position in prompt) of this wavefront
  const int qpos = r0 + col;         // the query this lane's column holds
  const int64_t qrow = (int64_t)q0 + qpos;
  const int64_t hq_row = (int64_t)p.num_q_heads * D;

  if (!ok) {  // offsets outside the buffers or an over-long prompt: row tile 0 writes NaN rows
    if (mt == 0) write_nan_rows<D>(p, q0, 0, L, h);
    return;
  }

  if (m0 >= L) return;

  const int n_end = p.causal ? min(L, m0 + kM) : L;
  const int n_tiles = (n_end + kN - 1) / kN;
  const uint32_t rowb = (uint32_t)p.num_kv_heads * D * 2u;  // bytes per key row

  PagedSrc src{};
  if constexpr (PAGED) {
    // page ids, kinds and scales of pages 0 .. 4 n_tiles - 1; an out-of-pool
    // id or unknown flag marks the row tile bad (its rows are written as NaN)
    if (!stage_page_meta(p, prompt, g, L, 4 * n_tiles, s_meta, s_scale, &s_bad)) {
      write_nan_rows<D>(p, q0, m0, min(L, m0 + kM), h);
      return;
    }
    src.kt = reinterpret_cast<const char*>(p.k_target) + (int64_t)g * D * 2;
    src.vt = reinterpret_cast<const char*>(p.v_target) + (int64_t)g * D * 2;
    src.kc = reinterpret_cast<const char*>(p.k_compact) + (int64_t)g * D * 2;
    src.vc = reinterpret_cast<const char*>(p.v_compact) + (int64_t)g * D;
    src.rowb = rowb;
    src.rowb8 = (uint32_t)p.num_kv_heads * D;
    src.range16 = (kPage - 1) * rowb + 2u * D;
    src.range8 = (kPage - 1) * src.rowb8 + (uint32_t)D;
  }

  // Q^T operand: lane holds Q[qpos][16ks + 8half .. +8] for each k-step.
  f16x8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qpos < L) {
      const uint4 x = *reinterpret_cast<const uint4*>(p.q + qrow * hq_row + (int64_t)h * D + 16 * ks + 8 * half);
      qb[ks] = __builtin_bit_cast(f16x8, x);
    } else {
      qb[ks] = f16x8{};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m = kNegBig, l = 0.f;

  // Per-lane load offsets.  V unit (kq, oc): workspace source kq = t % 16
  // (consecutive lanes take consecutive key quads); paged source kq = t / (D/8),
  // so a wavefront's units share two pages.
  constexpr int units = (kN / 4) * (D / 8);
  const bool v_active = threadIdx.x < units;
  const int vt_id = v_active ? threadIdx.x : 0;
  const int kq = PAGED ? vt_id / (D / 8) : vt_id % (kN / 4);
  const int oc = PAGED ? vt_id % (D / 8) : vt_id / (kN / 4);
  __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(nullptr, (short)0, 0, kBufferFlags);
  __amdgpu_buffer_rsrc_t vr = kr;
  uint32_t koff[KRegs<D>::KCH], voff[4];
  uint32_t pkoff = 0, pvoff16 = 0, pvoff8 = 0;
  if constexpr (PAGED) {
    // K chunk i: key t/(D/8) + (256/(D/8)) i, i.e. the same slot of tile page
    // 2i + wave/2; V rows 4(kq%4) .. +3 of tile page kq/4
    pkoff = (uint32_t)((threadIdx.x / (D / 8)) % kPage) * rowb + 16u * (threadIdx.x % (D / 8));
    pvoff16 = (uint32_t)(4 * (kq % 4)) * rowb + 16u * oc;
    pvoff8 = (uint32_t)(4 * (kq % 4)) * src.rowb8 + 8u * oc;
  } else {
    // workspace source: buffer descriptors over this prompt's K/V rows of KV head g
    const uint32_t span = (uint32_t)(L - 1) * rowb + D * 2u;
    const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)kv0 * p.num_kv_heads + g) * D * 2;
    const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)kv0 * p.num_kv_heads + g) * D * 2;
    kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, span, kBufferFlags);
    vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, span, kBufferFlags);
#pragma unroll
    for (int i = 0; i < KRegs<D>::KCH; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      koff[i] = (uint32_t)(idx / (D / 8)) * rowb + 16u * (idx % (D / 8));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)(4 * kq + i) * rowb + 16u * oc;
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  KRegs<D> kreg;
  VRegs vreg;
  vreg.v_codes = false;
  vreg.vscale = 1.0f;

  auto issue_k = [&](int t, const TileMetaRaw& tm) {
    if constexpr (PAGED) load_k_paged<D>(kreg, src, tm, wave_u, pkoff);
    else load_k<D>(kreg, kr, koff, (uint32_t)(t * kN) * rowb);
  };
  auto put_k = [&](SmemK<D>& sk) { store_k<D>(sk, kreg); };
  // QK^T A-operand offsets (halves) of k-step ks inside a 32-row key block
  uint32_t kro[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kro[ks] = (uint32_t)col * SmemK<D>::kStride + 8u * (uint32_t)half + 16u * (uint32_t)ks;
  auto issue_v = [&](int t, const TileMetaRaw& tm) {
    if constexpr (PAGED) load_v_paged<D>(vreg, src, tm, wave_u, lane, pvoff16, pvoff8);
    else load_v(vreg, vr, voff, (uint32_t)(t * kN) * rowb);
  };
  auto meta = [&](int t) {
    TileMetaRaw r{};
    if constexpr (PAGED) r = read_tile_meta(s_meta, s_scale, t);
    return r;
  };
  // Tiles 0 .. n_w - 1 hold keys this wavefront's rows can see (causal);
  // the later ones are staged for the other wavefronts but not computed.
  const int n_w = p.causal ? min(n_tiles, (r0 + 31) / kN + 1) : n_tiles;

  // S^T = K . Q^T of one 32-key block of a tile (8 MFMAs over the head dim)
  auto qk_block = [&](f32x16& sacc, const SmemK<D>& sk, int kb) {
    sacc = f32x16{};
    const f16* kp = &sk.k[kb * 32 * SmemK<D>::kStride];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(kp + kro[ks]);
      sacc = mfma32(a, qb[ks], sacc);
    }
  };

  // Causal diagonal / prompt-end mask on the raw scores of tile n0.
  auto mask_tile = [&](f32x16 (&sacc)[2], int n0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = n0 + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        const bool vis = key < L && (!p.causal || key <= qpos);
        sacc[kb][r] = vis ? sacc[kb][r] : -__builtin_inff();
      }
    }
  };

  // One compute step over tile t (scores CUR, already masked), with the
  // scores of tile t + 1 (NXT) computed on the matrix cores in the same
  // instruction stream: the running max of CUR interleaves with NXT's first
  // key block, the exponentials with its second key block and the P.V MFMAs
  // of CUR.  NXT may be garbage past the last computed tile (never used).
  auto step = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], const SmemK<D>& sk, const SmemV<D>& sv) {
    // running max (log2 units; scale > 0 keeps the max)
    qk_block(nxt[0], sk, 0);
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kb][r]);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    }
    mx = fmaxf(mx, shfl_xor(mx, 32)) * p.scale_log2;
    const float mnew = (mx > m + kTau) ? mx : m;
    if (__ballot(mnew != m)) {
      const float a = fast_exp2(m - mnew);
      l *= a;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= a;
      m = mnew;
    }
    qk_block(nxt[1], sk, 1);
    // P^T operand (fp16): PV k-block kk uses registers 8(kk%2)..+8 of block kk/2
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 pb;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float pv = fast_exp2(__builtin_fmaf(cur[kk / 2][8 * (kk % 2) + r], p.scale_log2, -m));
        l += pv;
        pb[r] = (f16)pv;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f16* vp = &sv.vt[(32 * db + col) * SmemV<D>::vStride];
        const int sw = vt_swz<PAGED>(32 * db + col);
        // key quads half + 4 kk (keys 16 kk + 4 half ..) and half + 4 kk + 2
        const uint2 lo = *reinterpret_cast<const uint2*>(vp + 4 * ((half + 4 * kk) ^ sw));
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 4 * ((half + 4 * kk + 2) ^ sw));
        const uint4 a4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[db] = mfma32(__builtin_bit_cast(f16x8, a4), pb, oacc[db]);
      }
    }
#pragma unroll
    for (int i = 0; i < KS + 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);  // three VALU
    }
  };

  // Prologue: K(0), V(0), K(1) into LDS, then S(0).  Paged source: a tile's
  // page metadata is read from LDS when its loads are issued, not carried a
  // tile ahead in registers.
  issue_k(0, meta(0));
  issue_v(0, meta(0));
  put_k(kbuf[0]);
  store_v<D, PAGED>(vbuf[0], vreg, kq, oc, v_active, PAGED ? L : kN);
  if (n_tiles > 1) {
    issue_k(1, meta(1));
    put_k(kbuf[1]);
  }
  __syncthreads();
  f32x16 sA[2], sB[2];
  qk_block(sA[0], kbuf[0], 0);
  qk_block(sA[1], kbuf[0], 1);
  // The first iteration stores K(2) into buffer 0: every wavefront must have
  // read K(0) from it first (later reuses are ordered by the per-tile barrier).
  __syncthreads();

  // Iteration t: loads of K(t+2) and V(t+1) are in flight while S(t+1) is
  // computed on the matrix cores and the softmax of S(t) runs on the vector
  // ALUs, then O += V(t) P(t); the staged tiles go to the buffers freed by
  // K(t) and V(t-1), and one barrier publishes them.
#define EKV_PREFILL_STEP(CUR, NXT)                                                              \
  {                                                                                             \
    if (it + 2 < n_tiles) issue_k(it + 2, meta(it + 2));                                        \
    if (it + 1 < n_tiles) issue_v(it + 1, meta(it + 1));                                        \
    if (it < n_w) {                                                                             \
      if ((p.causal && it * kN + kN - 1 > r0) || (it * kN + kN > L)) mask_tile(CUR, it * kN);   \
      step(CUR, NXT, kbuf[(it + 1) & 1], vbuf[it & 1]);                                         \
    }                                                                                           \
    if (it + 2 < n_tiles) put_k(kbuf[it & 1]);                                                  \
    if (it + 1 < n_tiles)                                                                       \
      store_v<D, PAGED>(vbuf[(it + 1) & 1], vreg, kq, oc, v_active, PAGED ? L - (it + 1) * kN : kN); \
    __syncthreads();                                                                            \
    if (++it >= n_tiles) break;                                                                 \
  }
  for (int it = 0; it < n_tiles;) {
    EKV_PREFILL_STEP(sA, sB)
    EKV_PREFILL_STEP(sB, sA)
  }
#undef EKV_PREFILL_STEP

  // normalize and store rows of this lane's column
  l += shfl_xor(l, 32);
  if (qpos >= L) return;
  const float inv = 1.0f / l;
  const int64_t obase = qrow * hq_row + (int64_t)h * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int d = 32 * db + 8 * rb + 4 * half;
      const float o0 = oacc[db][4 * rb + 0] * inv, o1 = oacc[db][4 * rb + 1] * inv;
      const float o2 = oacc[db][4 * rb + 2] * inv, o3 = oacc[db][4 * rb + 3] * inv;
      if (p.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d) = f32x4{o0, o1, o2, o3};
      } else {
        f16x2 a, b;
        a.x = (f16)o0; a.y = (f16)o1; b.x = (f16)o2; b.y = (f16)o3;
        *reinterpret_cast<uint2*>(static_cast<f16*>(p.out) + obase + d) = make_uint2(bits(a), bits(b));
      }
    }
  }
  if (p.lse && half == 0) p.lse[qrow * p.num_q_heads + h] = (m + log2f(l)) * kLn2;
}

// Head dim 128, workspace rows or pages: the same flash loop with the K and V
// tiles staged by buffer loads straight into LDS (no staging registers, no
// LDS stores for K and for fp16 V) and V^T operands read with gfx950
// transposing LDS reads.
//   LDS tiles are row-major, 256 B per key row, 16-byte chunks swizzled:
//   K chunk c of row r sits at chunk c ^ (r % 16): the 16 rows one
//   ds_read_b128 pass touches hit 16 distinct bank groups.  V chunk c of row
//   r sits at chunk c ^ 4 (r % 4): the 4 rows x 64 B one transposing read
//   pass touches hit 16 distinct bank groups.
//   Staging: each of the NW wavefronts moves 16 / NW K and as many V row
//   quads (1 KiB each) per tile; lane l writes bytes 16 l of its quad, i.e. row l / 16, swizzled
//   chunk l % 16, so it loads the source chunk that belongs there.  Rows past
//   the prompt are outside the descriptor range and arrive as zeros (paged
//   source: value rows; its key rows past the prompt are masked instead).
//   V^T operand: ds_read_b64_tr_b16 returns, in lane j of each 16-lane group,
//   element j % 4 of the 8-byte pieces addressed by lanes 4k + j / 4 (k =
//   0..3); lane i of the group addresses key row key0 + i / 4 at d offset
//   4 (i % 4), so lane j receives V[key0 + k][d0 + j] for k = 0..3: four keys
//   of one d, the A-operand layout of O^T = V^T P^T.
constexpr int kWsD = 128;
// Wavefronts per workgroup (32 query rows each), either source: 8 for
// prompts of at least kLongPrompt tokens (a staged tile serves 256 rows:
// 3-4% faster at 8 x 8192), 4 below (more workgroups: 11% faster at
// 32 x 512).  Paged source: a wavefront stages one page of each 64-key tile
// at 4 wavefronts, half a page at 8.
constexpr int kLongPrompt = 2048;
__host__ __device__ inline bool paged_route(const PrefillParams& p) { return p.page_table != nullptr; }


__device__ __forceinline__ uint2 lds_tr16(const f16* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Calls f(integral_constant<int, S>) for S = 0, 1, ...: a fully unrolled
// sequence whose step index is a compile-time constant in each call.
template <typename F, int... S>
__device__ __forceinline__ void unroll_steps(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}

// Head dim 128, both sources.  NW wavefronts of 32 query rows each share the
// staged K and V tiles; two wavefronts per SIMD (at most 256 VGPRs each).
// The loop runs over 32-key units u (half a 64-key tile) as a three-stage
// software pipeline: body u computes S(u + 2) = K Q^T and O += V(u)^T P(u)
// on the matrix cores while the vector ALUs take the exponentials of
// S(u + 1); none of the three depends on another.  A unit's exponentials
// are taken against the running max as it stands (deferred rescale): each
// lane sums its 16 weights of the unit, and only where some lane's sum
// exceeds 2^tau (a wave-uniform branch, rare once the max has settled)
// do the rows concerned take the unit's max, scale l and O by exp2(m_old -
// m_new) and take the unit's exponentials again.  Every weight is thus at
// most 2^tau, and each row sees the usual online-softmax recurrence with
// at most one rescale per unit (a row that keeps its max gets the factor
// 1 and the same weights, bit for bit).  P is rounded to fp16 for the P.V
// MFMAs and l sums those same fp16 values (v_dot2_f32_f16), so the
// normalisation divides by exactly the weights that multiplied V.
// Issue budget: one v_exp_f32 costs a wavefront about 8.5 clocks of issue
// and a plain VALU operation about 4.7, with no overlap between the two;
// a 32x32x16 MFMA keeps the matrix core busy 32 clocks.  A body has 16
// MFMAs, 16 exponentials and about 40 other VALU operations per
// wavefront, so the two wavefronts of a SIMD must interleave closely to
// keep the matrix cores fed: the steps of a full tile are fixed in order
// (see full_tile) with one exponential per MFMA.
template <int NW, bool PAGED>
__global__ __launch_bounds__(NW * kWave, 8 / NW) void prefill_pipe_kernel(PrefillParams p, int n_mtiles) {
  constexpr int RB = 1;  // 32-row blocks per wavefront (the compute loops allow more;
                         // the query and fp16 output staging assume one)
  constexpr int D = kWsD;
  constexpr int WR = 32 * RB;   // query rows per wavefront (RB 32-row blocks)
  constexpr int QUADS = 16 / NW;
  // paged source: a 64-key tile is 4 pages; each wavefront stages RPW rows
  // of page wave / PPW (a whole page at 4 wavefronts, half a page at 8)
  constexpr int PPW = NW / 4;
  constexpr int RPW = kPage / PPW;
  static_assert(!PAGED || NW == 4 || NW == 8, "paged staging: a page or half a page per wavefront");
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kN * D;
  // Four separate tile buffers: with the buffer known at compile time in the
  // main loop, the compiler can tell that a tile's LDS reads do not touch
  // the buffers the next tiles are being loaded into, and does not wait for
  // those loads before the reads.
  __shared__ __attribute__((aligned(1024))) f16 kb0[TILE];
  __shared__ __attribute__((aligned(1024))) f16 kb1[TILE];
  __shared__ __attribute__((aligned(1024))) f16 vb0[TILE];
  __shared__ __attribute__((aligned(1024))) f16 vb1[TILE];
  auto kbuf_of = [&](int b) -> f16* { return b ? kb1 : kb0; };
  auto vbuf_of = [&](int b) -> f16* { return b ? vb1 : vb0; };
  __shared__ __attribute__((aligned(16))) uint8_t vcodes[PAGED ? NW * RPW * D : 16];
  __shared__ __attribute__((aligned(16))) int s_meta[PAGED ? kMaxPromptPages : 4];
  __shared__ __attribute__((aligned(16))) float s_scale[PAGED ? kMaxPromptPages : 4];
  __shared__ int s_bad;
  // At 8 wavefronts (one workgroup per CU) each wavefront's 32 query rows
  // come in through this area: 8 KiB per wavefront, 64 KiB in all.
  constexpr bool QST = NW == 8;
  __shared__ __attribute__((aligned(1024))) f16 qst[QST ? NW * 32 * kWsD : 8];

  const int G = p.num_q_heads / p.num_kv_heads;
  const int HW = heads_per_workgroup(G, NW);  // query heads of this workgroup
  const int WB = WR * (NW / HW);              // positions of this workgroup
  const WorkItem wi = work_item_heads(p, n_mtiles, HW);
  const int prompt = wi.prompt, h0 = wi.h, mt = wi.mt;
  const int g = h0 / G;

  const int q0 = p.cu_seqlens_q[prompt];
  const int q1 = p.cu_seqlens_q[prompt + 1];
  if (q0 < 0 || q1 < q0 || q1 > p.q_rows) return;  // rows not addressable: nothing to write
  const int L = q1 - q0;
  const int m0 = mt * WB;
  const int kv0 = PAGED ? 0 : p.kv_start[prompt];
  const bool ok = PAGED ? (L <= p.max_len && L <= kMaxPromptPages * kPage &&
                           (int64_t)L <= (int64_t)p.pt_stride * kPage)
                        : (L <= p.max_len && kv0 >= 0 && (int64_t)kv0 + L <= p.kv_rows);
  if (!ok) {
    if (mt == 0)
      for (int hh = 0; hh < HW; ++hh) write_nan_rows<D>(p, q0, 0, L, h0 + hh);
    return;
  }
  if (m0 >= L) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  // wavefront w: head h0 + w % HW, block w / HW of 32 positions
  const int h = h0 + wave % HW;
  const int r0 = m0 + WR * (wave / HW);
  const int64_t hq_row = (int64_t)p.num_q_heads * D;
  const int n_end = p.causal ? min(L, m0 + WB) : L;
  const int n_tiles = (n_end + kN - 1) / kN;
  const uint32_t rowb = (uint32_t)p.num_kv_heads * D * 2u;
  const uint32_t rowb8 = (uint32_t)p.num_kv_heads * D;

  if constexpr (PAGED) {
    if (!stage_page_meta(p, prompt, g, L, 4 * n_tiles, s_meta, s_scale, &s_bad)) {
      for (int hh = 0; hh < HW; ++hh) write_nan_rows<D>(p, q0, m0, min(L, m0 + WB), h0 + hh);
      return;
    }
  }

  const uint32_t span = (uint32_t)(L - 1) * rowb + D * 2u;
  const char* kbase = reinterpret_cast<const char*>(PAGED ? p.k_target : p.k) + ((int64_t)kv0 * p.num_kv_heads + g) * D * 2;
  const char* vbase = reinterpret_cast<const char*>(PAGED ? p.v_target : p.v) + ((int64_t)kv0 * p.num_kv_heads + g) * D * 2;
  const char* kcbase = reinterpret_cast<const char*>(p.k_compact) + (int64_t)g * D * 2;
  const char* vcbase = reinterpret_cast<const char*>(p.v_compact) + (int64_t)g * D;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, span, kBufferFlags);

  uint32_t kso[QUADS], vso[QUADS];
#pragma unroll
  for (int j = 0; j < QUADS; ++j) {
    const int r = 4 * (QUADS * wave + j) + (lane >> 4), pc = lane & 15;
    const int rs = PAGED ? r % kPage : r;
    kso[j] = (uint32_t)rs * rowb + 16u * (uint32_t)(pc ^ (r & 15));
    vso[j] = (uint32_t)rs * rowb + 16u * (uint32_t)(pc ^ (4 * (r & 3)));
  }
  uint32_t cso[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) cso[c] = (uint32_t)(8 * c + (lane >> 3)) * rowb8 + 16u * (uint32_t)(lane & 7);
  auto page_meta = [&](int j) { return __builtin_amdgcn_readfirstlane(s_meta[j]); };
  auto stage_k = [&](int t, int b) {
    if constexpr (PAGED) {
      const int meta = page_meta(4 * t + wave / PPW);
      const char* base = ((meta & 1) ? kcbase : kbase) + (int64_t)(meta >> 1) * kPage * rowb;
      const __amdgpu_buffer_rsrc_t kd = __builtin_amdgcn_make_buffer_rsrc(
          (void*)base, (short)0, (kPage - 1) * rowb + D * 2u, kBufferFlags);
#pragma unroll
      for (int j = 0; j < QUADS; ++j) lds_dma16(kd, kbuf_of(b) + 4 * (QUADS * wave + j) * D, kso[j]);
    } else {
      const uint32_t to = (uint32_t)(t * kN) * rowb;
#pragma unroll
      for (int j = 0; j < QUADS; ++j) lds_dma16(kr, kbuf_of(b) + 4 * (QUADS * wave + j) * D, kso[j] + to);
    }
  };
  auto stage_v = [&](int t, int b) {
    if constexpr (PAGED) {
      const int pj = 4 * t + wave / PPW;
      const int meta = page_meta(pj);
      const uint32_t valid = (uint32_t)min(max(L - kPage * pj, 0), kPage);
      const int64_t phys = meta >> 1;
      if (meta & 1) {
        const __amdgpu_buffer_rsrc_t vd = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vcbase + phys * kPage * rowb8), (short)0, valid ? (valid - 1) * rowb8 + D : 0u, kBufferFlags);
#pragma unroll
        for (int c = 0; c < 2 / PPW; ++c)  // 1 KiB = 8 code rows per load
          lds_dma16(vd, reinterpret_cast<f16*>(&vcodes[wave * RPW * D + 1024 * c]),
                    cso[PPW == 1 ? c : (wave & 1)]);
      } else {
        const __amdgpu_buffer_rsrc_t vd = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vbase + phys * kPage * rowb), (short)0, valid ? (valid - 1) * rowb + D * 2u : 0u, kBufferFlags);
#pragma unroll
        for (int j = 0; j < QUADS; ++j) lds_dma16(vd, vbuf_of(b) + 4 * (QUADS * wave + j) * D, vso[j]);
      }
    } else {
      const uint32_t to = (uint32_t)(t * kN) * rowb;
#pragma unroll
      for (int j = 0; j < QUADS; ++j) lds_dma16(vr, vbuf_of(b) + 4 * (QUADS * wave + j) * D, vso[j] + to);
    }
  };
  auto put_v = [&](int t, int b) {
    if constexpr (PAGED) {
      const int pj = 4 * t + wave / PPW;
      if (page_meta(pj) & 1) {
        // lane l expands CPL codes of staged row l / SEGS, d CPL (l % SEGS) ..,
        // NCH 16-byte chunks of the fp16 row, one 8-byte code read and one
        // 16-byte store per chunk, in the order k = j + f(r) (mod NCH), f(r)
        // = r ^ (r >> log2 NCH): any 16 lanes (NCH consecutive rows) store to
        // 16 distinct chunk columns (distinct k modulo NCH; the row swizzle
        // keeps the index modulo NCH), and any 32 lanes (2 NCH rows of 128
        // codes) read from distinct banks (distinct k in the rows 256 bytes
        // apart), with the tile bytes and code reads of the plain order.
        constexpr int SEGS = kWave / RPW, CPL = D / SEGS, NCH = CPL / 8;
        constexpr int LNCH = NCH == 2 ? 1 : 2;
        static_assert(NCH == 2 || NCH == 4, "two or four chunks per lane");
        const float sc = rfl(s_scale[pj]);
        const int r = lane / SEGS, sg = lane % SEGS;
        const uint8_t* cs = &vcodes[wave * RPW * D + r * D + CPL * sg];
        const int R = RPW * wave + r;
        f16* row = vbuf_of(b) + R * D;
        const int sw = 4 * (R & 3);
        const int fr = r ^ (r >> LNCH);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int k = (j + fr) & (NCH - 1);
          const uint2 c = *reinterpret_cast<const uint2*>(cs + 8 * k);
          *reinterpret_cast<uint4*>(row + 8 * ((NCH * sg + k) ^ sw)) = expand8(c, sc);
        }
      }
    }
  };

  uint32_t kro[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kro[ks] = (uint32_t)col * D + 8u * (uint32_t)((2 * ks + half) ^ (col & 15));
  uint32_t vro[DB];
  {
    const int i = lane & 15, q16 = lane >> 4;
    const int row = 4 * (q16 >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * (q16 & 1) + ((i & 3) >> 1);
      vro[db] = (uint32_t)row * D + 8u * (uint32_t)(c ^ (4 * (row & 3))) + 4u * (uint32_t)(i & 1);
    }
  }

  // Q^T operands of both row blocks: query r0 + 32 rb + col
  f16x8 qb[RB][KS];
  f16* const qw = qst + (QST ? wave * 32 * D : 0);
  if constexpr (QST) {
    // Whole 256-byte rows by LDS-DMA, four rows per instruction, so each
    // load covers full cache lines (the operand layout below would touch 32
    // rows per instruction); lane l of load i fetches chunk (l % 16) ^ (row
    // % 16) of row 4 i + l / 16, so chunk k of a row sits at position k ^
    // (row % 16) and the operand reads below are bank-conflict free.  The
    // descriptor starts at this wavefront's first row (offsets stay within
    // 32 rows for any prompt length) and ends at the prompt's last row:
    // rows past it arrive as zeros.
    static_assert(RB == 1, "one 32-row block per wavefront");
    const int qrows = max(0, min(L - r0, WR));
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q + ((int64_t)q0 + r0) * hq_row + (int64_t)h * D), (short)0,
        qrows ? (uint32_t)(qrows - 1) * (uint32_t)hq_row * 2u + D * 2u : 0u, kBufferFlags);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint32_t c = (uint32_t)((lane & 15) ^ (r & 15));
      lds_dma16(qr, qw + i * 512, (uint32_t)r * (uint32_t)hq_row * 2u + 16u * c);
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qpos = r0 + 32 * rb + col;
      const int64_t qrow = (int64_t)q0 + qpos;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (qpos < L) {
          const uint4 x = *reinterpret_cast<const uint4*>(p.q + qrow * hq_row + (int64_t)h * D + 16 * ks + 8 * half);
          qb[rb][ks] = __builtin_bit_cast(f16x8, x);
        } else {
          qb[rb][ks] = f16x8{};
        }
      }
    }
  }
  f32x16 oacc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[rb][i] = f32x16{};
  // Running softmax state: max m (log2 units), row sum l (this lane's
  // half of the row's keys) and ls, the lane's sum of the weights of the
  // unit whose exponentials are being taken.  O and l always hold the
  // units before it against the current m.
  float m[RB], l[RB], ls[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    l[rb] = 0.f;
    ls[rb] = 0.f;
  }

  // Unit u = keys 32 u .. 32 u + 31 = half u % 2 of tile u / 2.
  // S(u) (prologue and last units; RB row blocks share each K operand).
  // All eight K operands are read before the first MFMA, so the chain waits
  // for one LDS latency instead of one per k-step.
  auto qk_unit = [&](f32x16 (&s)[RB], int u) {
    const f16* kp = kbuf_of((u >> 1) & 1) + (u & 1) * 32 * D;
    f16x8 a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = *reinterpret_cast<const f16x8*>(kp + kro[ks]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb] = mfma32(a[ks], qb[rb][ks], ks == 0 ? f32x16{} : s[rb]);
    }
  };
  auto unit_needs_mask = [&](int u) { return (p.causal && 32 * u + 31 > r0) || (32 * u + 32 > L); };
  // Called under a wave-uniform branch; the empty asm keeps the compiler from
  // turning that branch into selects executed for every unit.
  auto mask_unit = [&](f32x16 (&s)[RB], int u) {
    asm volatile("");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qpos = r0 + 32 * rb + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * u + 8 * (r / 4) + 4 * half + (r % 4);
        const bool vis = key < L && (!p.causal || key <= qpos);
        s[rb][r] = vis ? s[rb][r] : -__builtin_inff();
      }
    }
  };
  // Score maxima use the NaN-propagating maximum (v_maximum3_f32 on gfx950:
  // no canonicalising of the MFMA results first, as fmaxf needs); masked
  // scores are -inf, and a NaN score makes its row NaN either way.
  auto vmax = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  // The row max of a unit's scores in log2 units: a row's 32 scores lie in
  // two lanes, l and l ^ 32, 16 each (scale_log2 > 0 keeps the max).
  auto row_max = [&](const f32x16& s) {
    float x = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) x = vmax(x, s[r]);
    return vmax(x, shfl_xor(x, 32)) * p.scale_log2;
  };
  // P(u) = exp2(S(u) scale_log2 - m) as the fp16 B operands of the P.V
  // MFMAs; ls sums those same fp16 values in fp32, a pair per
  // v_dot2_f32_f16, so the normalisation divides by exactly the weights
  // that multiplied V.
  auto unit_exps = [&](const f32x16 (&s)[RB], f16x8 (&pn)[RB][2]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[rb][e], p.scale_log2, -m[rb]));
        const float p1 = fast_exp2(__builtin_fmaf(s[rb][e + 1], p.scale_log2, -m[rb]));
        const f16x2 pr = {(f16)p0, (f16)p1};
        ls[rb] = __builtin_amdgcn_fdot2(pr, f16x2{(f16)1.0f, (f16)1.0f}, e == 0 ? 0.f : ls[rb], false);
        pn[rb][e / 8][e % 8] = pr[0];
        pn[rb][e / 8][e % 8 + 1] = pr[1];
      }
    }
  };
  // O += V(u)^T P(u); each V^T operand feeds RB MFMAs
  auto pv_unit = [&](const f16x8 (&pb)[RB][2], int u) {
    const f16* vt = vbuf_of((u >> 1) & 1);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int kk = 2 * (u & 1) + k2;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint2 lo = lds_tr16(vt + vro[db] + 16 * kk * D);
        const uint2 hi = lds_tr16(vt + vro[db] + (16 * kk + 8) * D);
        const f16x8 a = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32(a, pb[rb][k2], oacc[rb][db]);
      }
    }
  };
  // Marks P as used here: keeps its exponentials in the body whose matrix
  // work hides them instead of letting them sink towards their first use.
  auto pin_p = [&](const f16x8 (&pb)[RB][2]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) asm volatile("" ::"v"(pb[rb][k2]));
  };
  // Ends the softmax of unit u + 1 once O holds P(u): a lane whose weights
  // of the unit sum past 2^tau (NaN sums do not) sends its row to the
  // unit's max; l and O are scaled by exp2(m_old - m_new) and the unit's
  // exponentials taken again (wave-uniform branch; the empty asm keeps it
  // a branch).  Rows that keep their max get the factor 1 and the same
  // weights.  Then l takes the unit's sum.
  auto settle = [&](const f32x16 (&s)[RB], f16x8 (&pn)[RB][2]) {
    bool over = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) over |= ls[rb] > kOver;
    if (__ballot(over) != 0) {
      asm volatile("");
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float lsp = shfl_xor(ls[rb], 32), xn = row_max(s[rb]);  // whole wavefront
        const bool row_over = (ls[rb] > kOver) | (lsp > kOver);
        const float mnew = row_over ? vmax(m[rb], xn) : m[rb];
        const float al = fast_exp2(m[rb] - mnew);
        m[rb] = mnew;
        l[rb] *= al;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[rb][i] *= al;
      }
      unit_exps(s, pn);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l[rb] += ls[rb];
  };

  // units this wavefront computes: up to its last row's diagonal and the
  // prompt's end (none if all its rows lie past the prompt)
  const int n_u = r0 >= L ? 0 : min(p.causal ? (r0 + WR - 1) / 32 + 1 : 2 * n_tiles, (L + 31) / 32);
  // Prologue: K(0), V(0), K(1) staged; S(0), its max, P(0); S(1) and its max.
  stage_k(0, 0);
  stage_v(0, 0);
  if (n_tiles > 1) stage_k(1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  put_v(0, 0);
  __syncthreads();
  if constexpr (QST) {  // each wavefront reads back only what its own loads wrote
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[0][ks] = *reinterpret_cast<const f16x8*>(qw + col * D + 8 * ((2 * ks + half) ^ (col & 15)));
  }
  f32x16 sA[RB], sB[RB];
  f16x8 pA[RB][2], pB[RB][2];
  if (n_u > 0) {
    qk_unit(sB, 0);
    if (unit_needs_mask(0)) mask_unit(sB, 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m[rb] = vmax(row_max(sB[rb]), kNegBig);  // l and O are zero
    unit_exps(sB, pA);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l[rb] = ls[rb];
    if (n_u > 1) {
      qk_unit(sA, 1);
      if (unit_needs_mask(1)) mask_unit(sA, 1);
    }
  }
  __syncthreads();

  // A tile whose two bodies u = 2 t and 2 t + 1 both have all their parts
  // runs as one explicitly ordered sequence of 32 steps (sched_barrier
  // fences keep the order).  Body b, step j issues
  //   j < 8:  the MFMA(s) of k-step j of S(u + 2)             (operand: K)
  //   j >= 8: the MFMA(s) of O += V(u)^T P(u) for (k2, db) =
  //           ((j - 8) / 4, (j - 8) % 4)                      (operand: V^T)
  // the LDS read of the operand of step j + kAhead and the exponential of
  // score j of S(u + 1) (fp16 pairs packed and summed at odd j); the
  // unit's softmax is settled at the body's end.  One transcendental and a few plain VALU operations per
  // MFMA keep the vector ALUs under the matrix cores' time.  Only the first
  // kAhead reads after the tile's barrier can stall the matrix cores.
  constexpr int kAhead = 3;
  // The tile parity (which of the two K and V buffers) is a compile-time
  // constant, so every LDS operand address is a fixed register plus an
  // immediate offset.
  auto full_tile = [&](int t, auto parity, auto masked) {
    constexpr int par = decltype(parity)::value;
    constexpr bool MASKED = decltype(masked)::value;
    const f16* kt = (par ^ 1) ? kb1 : kb0;  // K(t + 1): S(2t + 2) (keys 0..31), S(2t + 3)
    const f16* vt = par ? vb1 : vb0;        // V(t): P(2t) (kk 0, 1), P(2t + 1) (kk 2, 3)
    auto operand = [&](int s) -> f16x8 {
      const int b = s >> 4, j = s & 15;
      if (j < 8) return *reinterpret_cast<const f16x8*>(kt + b * 32 * D + kro[j]);
      const int kk = 2 * b + ((j - 8) >> 2), db = (j - 8) & 3;
      const uint2 lo = lds_tr16(vt + vro[db] + 16 * kk * D);
      const uint2 hi = lds_tr16(vt + vro[db] + (16 * kk + 8) * D);
      return __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    f16x8 ring[kAhead + 1];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) ring[s] = operand(s);
    float pe[RB];
    auto step = [&](auto step_index) {
      constexpr int s = decltype(step_index)::value;
      constexpr int b = s >> 4, j = s & 15;
      f32x16 (&sn)[RB] = b == 0 ? sB : sA;    // S(u + 2), produced
      f32x16 (&sc)[RB] = b == 0 ? sA : sB;    // S(u + 1), exponentials
      f16x8 (&pc)[RB][2] = b == 0 ? pA : pB;  // P(u), consumed by P.V
      f16x8 (&pn)[RB][2] = b == 0 ? pB : pA;  // P(u + 1), produced
      if constexpr (s + kAhead < 32) ring[(s + kAhead) % (kAhead + 1)] = operand(s + kAhead);
      const f16x8 a = ring[s % (kAhead + 1)];
      if constexpr (j < 8) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sn[rb] = mfma32(a, qb[rb][j], j == 0 ? f32x16{} : sn[rb]);
      } else {
        constexpr int k2 = (j - 8) >> 2, db = (j - 8) & 3;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32(a, pc[rb][k2], oacc[rb][db]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float pv = fast_exp2(__builtin_fmaf(sc[rb][j], p.scale_log2, -m[rb]));
        if constexpr ((j & 1) == 0) {
          pe[rb] = pv;
        } else {
          const f16x2 pr = {(f16)pe[rb], (f16)pv};
          ls[rb] = __builtin_amdgcn_fdot2(pr, f16x2{(f16)1.0f, (f16)1.0f}, j == 1 ? 0.f : ls[rb], false);
          pn[rb][j / 8][(j % 8) - 1] = pr[0];
          pn[rb][j / 8][j % 8] = pr[1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (j == 7) {
        // the first eight exponentials stay ahead of the mask branch
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) asm volatile("" ::"v"(ls[rb]), "v"(pn[rb][0]));
        if constexpr (MASKED)
          if (unit_needs_mask(2 * t + b + 2)) mask_unit(sn, 2 * t + b + 2);
      } else if constexpr (j == 15) {
        pin_p(pn);
        settle(sc, pn);
      }
    };
    unroll_steps(step, std::make_integer_sequence<int, 32>{});
  };
  // The same for the last units of the wavefront (some parts absent).
#define EKV_PIPE_TAIL(U, SC, SN, PC, PN)                                  \
  if ((U) < n_u) {                                                        \
    if ((U) + 1 < n_u) unit_exps(SC, PN);                                 \
    if ((U) + 2 < n_u) {                                                  \
      qk_unit(SN, (U) + 2);                                               \
      if (unit_needs_mask((U) + 2)) mask_unit(SN, (U) + 2);               \
    }                                                                     \
    pv_unit(PC, (U));                                                     \
    if ((U) + 1 < n_u) settle(SC, PN);                                    \
  }
  // Tiles whose two bodies are both complete form the main loop; every tile
  // (either loop) stages K(t + 2) and V(t + 1) and ends at the barrier.
  const int n_full = max(0, min(n_tiles, (n_u - 2) / 2));
  int it = 0;
  auto main_tile = [&](int t, auto parity, auto masked) {
    constexpr int par = decltype(parity)::value;
    if (t + 2 < n_tiles) stage_k(t + 2, par);
    if (t + 1 < n_tiles) stage_v(t + 1, par ^ 1);
    full_tile(t, parity, masked);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (t + 1 < n_tiles) put_v(t + 1, par ^ 1);
    __syncthreads();
  };
  // Whether a unit needs its mask only grows with the unit (the diagonal,
  // then the prompt's end), so at 8 wavefronts the full tiles before the
  // first such unit run a copy of the tile without the mask test and its
  // branch (1-3% on long prompts; at 4 wavefronts the second copy costs
  // registers and is slower).
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (NW == 8) {
    const int first_masked = min(p.causal ? r0 / 32 : L / 32, L / 32);
    const int n_clean = min(n_full, max(0, (first_masked - 2) / 2));  // full tiles t with 2 t + 3 < first_masked
    for (; it + 1 < n_clean; it += 2) {
      main_tile(it, I0{}, std::false_type{});
      main_tile(it + 1, I1{}, std::false_type{});
    }
  }
  for (; it + 1 < n_full; it += 2) {
    main_tile(it, I0{}, std::true_type{});
    main_tile(it + 1, I1{}, std::true_type{});
  }
  if (it < n_full) {
    main_tile(it, I0{}, std::true_type{});
    ++it;
  }
  for (; it < n_tiles; ++it) {
    if (it + 2 < n_tiles) stage_k(it + 2, it & 1);
    if (it + 1 < n_tiles) stage_v(it + 1, (it + 1) & 1);
    EKV_PIPE_TAIL(2 * it, sA, sB, pA, pB)
    EKV_PIPE_TAIL(2 * it + 1, sB, sA, pB, pA)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (it + 1 < n_tiles) put_v(it + 1, (it + 1) & 1);
    __syncthreads();
  }
#undef EKV_PIPE_TAIL

  if (!p.out_f32) {
    // fp16 rows go out through LDS so that each store instruction writes
    // four whole 256-byte rows (written from the accumulator layout, each
    // store instruction would touch 32 rows, 16 bytes each, and the
    // epilogue took 2.6x as long).  The tile buffers are free after the last
    // barrier: 8 KiB per wavefront, 16-byte chunks XOR-swizzled by row; each
    // wavefront reads back only its own rows.  fp32 rows keep direct stores.
    static_assert(RB == 1, "one 32-row block per wavefront");
    f16* ost = ((wave >> 1) == 0 ? kb0 : (wave >> 1) == 1 ? kb1 : (wave >> 1) == 2 ? vb0 : vb1) + (wave & 1) * 32 * D;
    l[0] += shfl_xor(l[0], 32);
    const int qpos = r0 + col;
    const float inv = 1.0f / l[0];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f16x2 a, b;
        a.x = (f16)(oacc[0][db][4 * rq + 0] * inv); a.y = (f16)(oacc[0][db][4 * rq + 1] * inv);
        b.x = (f16)(oacc[0][db][4 * rq + 2] * inv); b.y = (f16)(oacc[0][db][4 * rq + 3] * inv);
        *reinterpret_cast<uint2*>(ost + col * D + 8 * ((4 * db + rq) ^ (col & 15)) + 4 * half) =
            make_uint2(bits(a), bits(b));
      }
    }
    if (p.lse && half == 0 && qpos < L)
      p.lse[((int64_t)q0 + qpos) * p.num_q_heads + h] = (m[0] + log2f(l[0])) * kLn2;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const uint4 v = *reinterpret_cast<const uint4*>(ost + r * D + 8 * (c ^ (r & 15)));
      if (r0 + r < L)
        *reinterpret_cast<uint4*>(static_cast<f16*>(p.out) + ((int64_t)q0 + r0 + r) * hq_row + (int64_t)h * D + 8 * c) = v;
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l[rb] += shfl_xor(l[rb], 32);
    const int qpos = r0 + 32 * rb + col;
    if (qpos >= L) continue;
    const int64_t qrow = (int64_t)q0 + qpos;
    const float inv = 1.0f / l[rb];
    const int64_t obase = qrow * hq_row + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * db + 8 * rq + 4 * half;
        const float o0 = oacc[rb][db][4 * rq + 0] * inv, o1 = oacc[rb][db][4 * rq + 1] * inv;
        const float o2 = oacc[rb][db][4 * rq + 2] * inv, o3 = oacc[rb][db][4 * rq + 3] * inv;
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d) = f32x4{o0, o1, o2, o3};
        } else {
          f16x2 a, b;
          a.x = (f16)o0; a.y = (f16)o1; b.x = (f16)o2; b.y = (f16)o3;
          *reinterpret_cast<uint2*>(static_cast<f16*>(p.out) + obase + d) = make_uint2(bits(a), bits(b));
        }
      }
    }
    if (p.lse && half == 0) p.lse[qrow * p.num_q_heads + h] = (m[rb] + log2f(l[rb])) * kLn2;
  }
}
}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.n_prompts == 0 || p.max_len == 0) return hipSuccess;
  const int n_mtiles = (p.max_len + kM - 1) / kM;
  const int64_t blocks = (int64_t)n_mtiles * p.num_q_heads * p.n_prompts;
  const dim3 grid((unsigned)blocks), block(kThreads);
  const bool paged = paged_route(p);
  if (paged && p.max_len > kMaxPromptPages * kPage) return hipErrorInvalidValue;
  if (p.head_dim == kWsD) {
    const int nw = p.max_len >= kLongPrompt ? 8 : 4;
    const int hw = heads_per_workgroup(p.num_q_heads / p.num_kv_heads, nw);
    const int wb = 32 * (nw / hw);
    const int n_mt = (p.max_len + wb - 1) / wb;
    const dim3 g((unsigned)((int64_t)n_mt * (p.num_q_heads / hw) * p.n_prompts)), blk(nw * kWave);
    if (paged && nw == 8) hipLaunchKernelGGL((prefill_pipe_kernel<8, true>), g, blk, 0, stream, p, n_mt);
    else if (paged) hipLaunchKernelGGL((prefill_pipe_kernel<4, true>), g, blk, 0, stream, p, n_mt);
    else if (nw == 8) hipLaunchKernelGGL((prefill_pipe_kernel<8, false>), g, blk, 0, stream, p, n_mt);
    else hipLaunchKernelGGL((prefill_pipe_kernel<4, false>), g, blk, 0, stream, p, n_mt);
    return hipGetLastError();
  }
  if (p.head_dim == 64) {
    if (paged) hipLaunchKernelGGL((prefill_kernel<64, true>), grid, block, 0, stream, p, n_mtiles);
    else hipLaunchKernelGGL((prefill_kernel<64, false>), grid, block, 0, stream, p, n_mtiles);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ekv

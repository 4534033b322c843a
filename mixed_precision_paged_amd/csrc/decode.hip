// GQA decode attention over a mixed-fidelity paged KV cache (split-K + merge).
//
// Sources: "Does Execution Require Target KV Fidelity?" (ElasticKV), section
// 3.2 and appendix B.3: TARGET and compact pages execute in one batch behind
// one output interface, and compact values are expanded into the native
// 16-bit datatype in registers without materializing TARGET.  "Memory-Traffic
// Saturation in Autoregressive Transformer Decode", section "What changes in
// vLLM's prefill routing?": decode reads persistent FP16 keys and FP8 E4M3
// values, NHD layout, page size 16, and value scales apply in attention;
// "Kernel families and hardware constraints" notes: place the scale in
// software, advance the online softmax tile by tile.
//
// Work decomposition (HBM-bound: every K/V byte is read exactly once):
//   workgroup = (split of pages, KV head g, sequence b); its wavefronts take
//   the split's pages round-robin, one page (16 tokens x D) at a time, with
//   the next page's loads in flight while the current one computes.  Page
//   ids, flags and value scales of the split are staged in LDS once.
//   Loads go through a buffer descriptor that spans exactly one page of one
//   KV head.
//   QK^T: v_mfma_f32_16x16x32_f16 computes S^T = K Q^T with the page's 16
//   tokens as rows and the G = Hq/Hkv query heads as columns (padded to 16),
//   so the G heads share every K/V load.
//   Softmax: online, in log2 units; the running max is raised only when a
//   page max exceeds it by more than kTau (exact: softmax is shift invariant;
//   it only skips rescales).
//   PV: the scores are the A operand of v_mfma_f32_16x16x16f16 with V as B;
//   P goes in as an fp16 hi + lo pair (two MFMAs), p = hi + lo to ~22 bits.
//   Compact pages expand their E4M3 bytes in registers with the gfx950
//   scaled conversion by the power-of-two part 2^e of the page-head scale
//   (exact: code * 2^e is an fp16 value for e in [-15, 7]; a scale outside
//   that range expands by the nearest end of it and rescales the page's
//   P.V products in fp32 by the remaining power of two); the mantissa part
//   f of the scale multiplies p in fp32.  Both kinds meet in one fp16-value PV path.  The
//   flag is per page, so the branch is wavefront-uniform.
//   End of split: wavefronts merge through LDS.  One split per sequence: the
//   workgroup writes the normalized output and LSE.  Several: it writes
//   (max, sum, unnormalized acc) partials and the merge kernel combines them:
//   M = max m_s, L = sum l_s 2^(m_s-M), o = sum acc_s 2^(m_s-M) / L,
//   lse = (M + log2 L) ln 2.
//   Ragged batches (balanced plan): every workgroup takes an equal,
//   contiguous share of the batch's page-heads in (sequence, KV head, page)
//   order, found by a binary search over prefix sums of the page counts; a
//   share may cut (sequence, head) ranges at either end and span several, and
//   each range it holds runs through the same page loop.  A range that is a
//   whole (sequence, head) is written directly, the rest go through the
//   merge, which finds a cut range's pieces in the workgroups its share
//   spans.
#include "ekv_device.hpp"
#include "ekv_internal.hpp"

namespace ekv {
namespace {

constexpr float kTau = 8.0f;          // deferred-rescale threshold (log2 units)
constexpr float kNegBig = -1.0e30f;   // "no token yet" running max
constexpr bool kHeadMajorGrid = true; // launch order: the KV heads of one (sequence, split) adjacent
constexpr int kMaxSplitPages = 512;   // pages per split (metadata staged in LDS)
constexpr int kBalancedRound = 256;     // balanced plan: workgroups per round (one per CU)
constexpr int kBalancedMaxPages = 512;  // balanced plan: pages per range (LDS stage)
constexpr int kBalancedWaves = 8;       // balanced plan: wavefronts per workgroup
constexpr int kNonTemporal = 2;      // buffer-load cache policy bit: non-temporal (streamed once)
constexpr int kKAux = 0;              // cache policy of K page loads
constexpr int kVAux = kNonTemporal;   // cache policy of V page loads
constexpr int kBaseKAux = 0;          // cache policy of BASE K page loads
constexpr int kSlots = 2;             // register page buffers per wavefront (pages in flight + 1)
constexpr int kMinWaves = 2;          // occupancy bound (wavefronts per SIMD) for G*D < 1024
constexpr int kExpLo = -15;           // code * 2^x is exact in fp16 for every E4M3 code iff
constexpr int kExpHi = 7;             //   x in [kExpLo, kExpHi] (2^-9 * 2^-15 = 2^-24; 448 * 2^7 < 65504)
constexpr int kMaxShift = 60;         // bound of the fp32 rescale of acc for out-of-range scales

template <int D>
struct PageRegs {
  f16x8 k[D / 32];       // K[token l%16][32kb + 8(l/16) .. +8]: MFMA A operand of S^T = K Q^T
  uint32_t v[4][D / 32]; // V rows of tokens 4(l/16)+i at d = (D/16)(l%16) .. +D/16 (fp16 pairs;
                         // COMPACT: the first D/64 dwords of a row hold its D/16 E4M3 bytes)
};

// One prefetch slot: a page's K/V registers plus its uniform metadata.
template <int D>
struct Slot {
  PageRegs<D> r;
  int kind;
  float scale;
  bool ok;
};

// Loads one page's K and V rows of this lane with buffer loads.  The buffer
// descriptors (wavefront-uniform, SGPRs) cover exactly one page of one KV
// head, so the hardware range check keeps every access inside that page.
// `kqoff` (token l%16, 16 B chunk l/16) and `voff` (token 4(l/16), d chunk
// l%16) are per-lane byte offsets; the token step of V goes in the scalar
// offset.  Each V load instruction covers 4 whole token rows.
// BASE pages (ElasticKV high bytes; only in the HAS_BASE variants) hold one
// byte per K element: a lane's 8 K values of a k-step are 8 bytes at `kqoff8`,
// loaded into the low half of r.k[kb] and expanded before the MFMA; their V
// bytes take the compact path's byte layout.
template <int D, bool HAS_BASE, int KAUX, int VAUX>
__device__ __forceinline__ void load_page(PageRegs<D>& r, int kind, const char* kbase,
                                          const char* vbase, uint32_t kbytes, uint32_t vbytes,
                                          uint32_t kqoff, uint32_t kqoff8, uint32_t voff16, uint32_t voff8,
                                          uint32_t krow, uint32_t vrow) {
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, kbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, vbytes, kBufferFlags);
  if (HAS_BASE && kind == 2) {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(kr, kqoff8 + 32u * kb, 0, kBaseKAux);
      r.k[kb] = __builtin_bit_cast(f16x8, u32x4{a.x, a.y, 0u, 0u});
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      r.k[kb] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, kqoff + 64u * kb, 0, KAUX));
  }
  if constexpr (HAS_BASE) {
    // Same load sequence for every kind (and for no page: range-0
    // descriptors), so the wait before a page's compute leaves the next
    // page's loads in flight: V rows as two halves of D/16 bytes, an fp16
    // page filling both, a byte page (codes, BASE) the low one while the high
    // one reads zeros.  Measured: 15% faster on BASE-heavy batches, 1-4%
    // slower on TARGET/COMPACT ones, hence only in the BASE variants.
    constexpr int HW = D / 64;
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, kind != 0 ? 0u : vbytes, kBufferFlags);
    if (kind != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (HW == 2) {
          const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(vr, voff8, i * vrow, VAUX);
          r.v[i][0] = a.x; r.v[i][1] = a.y;
        } else {
          r.v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, voff8, i * vrow, 0);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (HW == 2) {
          const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(vr, voff16, i * krow, VAUX);
          r.v[i][0] = a.x; r.v[i][1] = a.y;
        } else {
          r.v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, voff16, i * krow, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (HW == 2) {
        const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(hr, voff16 + 8u, i * krow, VAUX);
        r.v[i][2] = b.x; r.v[i][3] = b.y;
      } else {
        r.v[i][1] = __builtin_amdgcn_raw_buffer_load_b32(hr, voff16 + 4u, i * krow, 0);
      }
    }
  } else if (kind == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (D == 128) {
        const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(vr, voff16, i * krow, VAUX);
        r.v[i][0] = y.x; r.v[i][1] = y.y; r.v[i][2] = y.z; r.v[i][3] = y.w;
      } else {
        const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(vr, voff16, i * krow, 0);
        r.v[i][0] = y.x; r.v[i][1] = y.y;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (D == 128) {
        const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(vr, voff8, i * vrow, VAUX);
        r.v[i][0] = y.x; r.v[i][1] = y.y; r.v[i][2] = 0u; r.v[i][3] = 0u;
      } else {
        r.v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, voff8, i * vrow, 0);
        r.v[i][1] = 0u;
      }
    }
  }
}

template <int D, int G>
struct State {
  f16x8 qb[D / 32];      // Q[head l%16][32kb + 8(l/16) .. +8]: MFMA B operand (0 for head >= G)
  float m, l;            // running max (log2 units) and partial sum of head l%16 (this lane's tokens)
  f32x4 acc[D / 16];     // O[head 4(l/16)+i][d = (D/16)(l%16) + e] * 2^-aexp in acc[e][i]
  int aexp;              // wavefront-uniform power-of-two offset of acc (0 unless scales are extreme)
};

__device__ __forceinline__ f16x4 pack4(float a, float b, float c, float d) {
  return f16x4{(f16)a, (f16)b, (f16)c, (f16)d};
}

// Eight BASE bytes (two words) -> eight fp16 values: each byte in the high
// position of its 16 bits, the low byte zero (selector 0x0C gives 0x00).
__device__ __forceinline__ f16x8 base_expand(f16x8 raw) {
  const u32x4 w = __builtin_bit_cast(u32x4, raw);
  return __builtin_bit_cast(f16x8, u32x4{perm(w.x, w.x, 0x010C000Cu), perm(w.x, w.x, 0x030C020Cu),
                                         perm(w.y, w.y, 0x010C000Cu), perm(w.y, w.y, 0x030C020Cu)});
}

template <int D, int G, bool HAS_BASE>
__device__ __forceinline__ void process_page(State<D, G>& st, PageRegs<D>& r, const DecodeParams& p,
                                             int kind, float scale, int pg, int len, int lane) {
  constexpr int NE = D / 16;  // PV MFMAs (d columns per lane)
  const int tq = lane >> 4;
  // Compact scale s = 2^sexp * f, f in [1, 2): the conversion applies a power of two, p
  // carries f.  code * 2^x is an fp16 value for every E4M3 code only for x in [kExpLo,
  // kExpHi], so the conversion gets x = sexp - shift in that range and the page's P.V
  // products need the factor 2^shift.  acc is kept as true value * 2^-st.aexp; a page
  // whose shift differs from st.aexp first rescales acc by 2^(st.aexp - shift) (a power
  // of two: exact while acc stays normal) and sets st.aexp = shift.  Scales derived from fp16 values (the cache writer) have sexp in
  // [-33, 7]; |shift| is bounded by kMaxShift.  (Scales are positive normal fp32 values.)
  const uint32_t sbits = kind == 1 ? __builtin_bit_cast(uint32_t, scale) : 0x3F800000u;
  const int sexp = (int)((sbits >> 23) & 0xFFu) - 127;
  const int shift = sexp < kExpLo   ? max(sexp - kExpLo, -kMaxShift)
                    : sexp > kExpHi ? min(sexp - kExpHi, kMaxShift)
                                    : 0;
  const float s_pow2 = as_f32((uint32_t)(sexp - shift + 127) << 23);
  const float s_frac = as_f32((sbits & 0x807FFFFFu) | 0x3F800000u);
  const bool partial = pg * kPage + kPage > len;  // wavefront-uniform

  // S^T = K . Q^T on the matrix cores: lane l gets the scores of head l%16 for
  // tokens 4(l/16)+i of the page (i < 4).
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (HAS_BASE && kind == 2) {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(base_expand(r.k[kb]), st.qb[kb], sacc, 0, 0, 0);
  } else {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(r.k[kb], st.qb[kb], sacc, 0, 0, 0);
  }
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = sacc[i] * p.scale_log2;
  if (partial) {  // last page of the sequence: drop slots >= len (their contents are undefined)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = pg * kPage + 4 * tq + i < len;
      x[i] = ok ? x[i] : -__builtin_inff();
#pragma unroll
      for (int w = 0; w < D / 32; ++w) r.v[i][w] = ok ? r.v[i][w] : 0u;
    }
  }

  // Online softmax per head; the page max spans the 4 lanes holding the head.
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  const float mnew = (mx > st.m + kTau) ? mx : st.m;
  if (__ballot(mnew != st.m)) {
    const float a = fast_exp2(st.m - mnew);  // 1 when unchanged, 0 from kNegBig
    st.l *= a;
    // acc rows are heads 4(l/16)+i: fetch their factors from lanes 4(l/16)+i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (4 * tq + i), __builtin_bit_cast(int, a)));
#pragma unroll
      for (int e = 0; e < NE; ++e) st.acc[e][i] *= ai;
    }
    st.m = mnew;
  }
  if (shift != st.aexp) {  // wavefront-uniform; only for page-head scales outside the exact range
    const float k = as_f32((uint32_t)(st.aexp - shift + 127) << 23);  // 2^(aexp - shift), exact
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[e][i] *= k;
    st.aexp = shift;
  }
  float pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv[i] = fast_exp2(x[i] - st.m);
    st.l += pv[i];
    pv[i] *= s_frac;
  }
  // P (A operand of the 16x16x16 P.V MFMA) in two fp16 parts: p = hi + lo to ~22 bits.
  const f16x4 phi = pack4(pv[0], pv[1], pv[2], pv[3]);
  const f16x4 plo = pack4(pv[0] - (float)phi[0], pv[1] - (float)phi[1], pv[2] - (float)phi[2],
                          pv[3] - (float)phi[3]);

  // V operands: for column set e, lane l holds V[tokens 4(l/16)..+3][d = (D/16)(l%16) + e].
  f16x4 vb[NE];
  if (kind == 0) {
#pragma unroll
    for (int w = 0; w < NE / 2; ++w) {
      const uint32_t e0 = perm(r.v[1][w], r.v[0][w], 0x05040100u), e1 = perm(r.v[3][w], r.v[2][w], 0x05040100u);
      const uint32_t o0 = perm(r.v[1][w], r.v[0][w], 0x07060302u), o1 = perm(r.v[3][w], r.v[2][w], 0x07060302u);
      vb[2 * w] = __builtin_bit_cast(f16x4, u32x2{e0, e1});
      vb[2 * w + 1] = __builtin_bit_cast(f16x4, u32x2{o0, o1});
    }
  } else if (HAS_BASE && kind == 2) {
    // BASE bytes: column c of dword w is d = 4w + c; each token's byte goes to
    // the high position of its fp16 (tokens 0, 1 from rows 0, 1; 2, 3 from 2, 3)
#pragma unroll
    for (int w = 0; w < NE / 4; ++w) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t sel = 0x040C000Cu + 0x01000100u * c;
        vb[4 * w + c] = __builtin_bit_cast(f16x4, u32x2{perm(r.v[1][w], r.v[0][w], sel),
                                                        perm(r.v[3][w], r.v[2][w], sel)});
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < NE / 4; ++w) {
      const uint32_t a01 = perm(r.v[1][w], r.v[0][w], 0x05010400u), a23 = perm(r.v[3][w], r.v[2][w], 0x05010400u);
      const uint32_t b01 = perm(r.v[1][w], r.v[0][w], 0x07030602u), b23 = perm(r.v[3][w], r.v[2][w], 0x07030602u);
      vb[4 * w + 0] = __builtin_bit_cast(f16x4, u32x2{bits(e4m3x2_scaled_f16(a01, s_pow2, false)), bits(e4m3x2_scaled_f16(a23, s_pow2, false))});
      vb[4 * w + 1] = __builtin_bit_cast(f16x4, u32x2{bits(e4m3x2_scaled_f16(a01, s_pow2, true)), bits(e4m3x2_scaled_f16(a23, s_pow2, true))});
      vb[4 * w + 2] = __builtin_bit_cast(f16x4, u32x2{bits(e4m3x2_scaled_f16(b01, s_pow2, false)), bits(e4m3x2_scaled_f16(b23, s_pow2, false))});
      vb[4 * w + 3] = __builtin_bit_cast(f16x4, u32x2{bits(e4m3x2_scaled_f16(b01, s_pow2, true)), bits(e4m3x2_scaled_f16(b23, s_pow2, true))});
    }
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    st.acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(phi, vb[e], st.acc[e], 0, 0, 0);
    st.acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(plo, vb[e], st.acc[e], 0, 0, 0);
  }
}

// Output rows of the G query heads of KV head g in sequence b when the
// sequence is empty: out 0, lse -inf (single-split launches only).
template <int D, int G>
__device__ void write_empty_rows(const DecodeParams& p, int b, int g) {
  const int64_t row0 = (int64_t)b * p.num_q_heads + g * G;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    if (p.out_f32) static_cast<float*>(p.out)[row0 * D + i] = 0.f;
    else static_cast<f16*>(p.out)[row0 * D + i] = (f16)0.f;
  }
  if (p.lse && (int)threadIdx.x < G) p.lse[row0 + threadIdx.x] = -__builtin_inff();
}

// LDS of one workgroup of NW wavefronts working on one piece of a sequence.
template <int D, int G, int NW, int MAXP = kMaxSplitPages>
struct PieceSmem {
  static constexpr int kMaxPages = MAXP;
  float acc[NW][G][D];
  float m[NW][G];
  float l[NW][G];
  int bad[NW];
  int meta[MAXP];
  float scale[MAXP];  // page-head value scale of each compact page of the piece (1 otherwise)
};

// MODE 0: every page has kind p.uniform_kind (no flag table); 1: per-page flags
// TARGET/COMPACT; 2: per-page flags that may also be BASE (the batch-level
// BASE indicator is set); 3: structured TARGET-BASE-TARGET layout: logical
// pages [base_bounds[b][0], base_bounds[b][1]) of sequence b are BASE, all
// others TARGET, with no flag table.
//
// Attention of the G query heads of KV head g of sequence b (length len) over
// its logical pages [pbeg, pend) (at most SM::kMaxPages): the NW wavefronts
// take the pages round-robin and leave their (max, sum, unnormalized acc) and
// bad-page flags in sm, published by a barrier.  The caller must not reuse sm
// before every wavefront has read what it needs (a barrier).
template <int D, int G, int MODE, int NW, int KAUX, int VAUX, class SM>
__device__ __forceinline__ void run_piece(const DecodeParams& p, SM& sm, int b, int g, int len,
                                          int pbeg, int pend, int lane, int wave) {
  constexpr int kThreads = NW * kWave;
  constexpr int kWaves = NW;
  constexpr bool FLAGS = MODE == 1 || MODE == 2;
  constexpr bool HAS_BASE = MODE >= 2;
  constexpr int KBITS = HAS_BASE ? 2 : 1;  // kind bits in the staged page metadata
  constexpr int NE = D / 16;
  State<D, G> st;
  {
    const int qh = lane & 15, qc = lane >> 4;
    const uint16_t* qp = p.q + ((int64_t)b * p.num_q_heads + g * G + (qh < G ? qh : 0)) * D + 8 * qc;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      st.qb[kb] = qh < G ? __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(qp + 32 * kb)) : f16x8{};
  }
  st.m = kNegBig;
  st.l = 0.f;
  st.aexp = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) st.acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage this split's page metadata in LDS once: (phys << KBITS | kind), or
  // -1 for an out-of-range id or unknown flag, and each compact page's scale.
  // Per-page reads are then LDS reads, which never wait on the vector-memory
  // counter of in-flight pages.
  // A BASE page id names half (id & 1) of TARGET block id >> 1.
  {
    const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride;
    const uint8_t* fl = FLAGS ? p.fidelity + (int64_t)b * p.pt_stride : nullptr;
    const int blo = MODE == 3 ? p.base_bounds[2 * b] : 0;
    const int bhi = MODE == 3 ? p.base_bounds[2 * b + 1] : 0;
    for (int i = threadIdx.x; i < pend - pbeg; i += kThreads) {
      const int phys = pt[pbeg + i];
      const int j = pbeg + i;
      const int kind = FLAGS ? (int)fl[j] : MODE == 3 ? (j >= blo && j < bhi ? 2 : 0) : p.uniform_kind;
      const bool ok = (kind == 0 && (unsigned)phys < (unsigned)p.n_target) ||
                      (kind == 1 && (unsigned)phys < (unsigned)p.n_compact) ||
                      (HAS_BASE && kind == 2 && (unsigned)phys < 2u * (unsigned)p.n_target);
      sm.meta[i] = ok ? (phys << KBITS) | kind : -1;
      sm.scale[i] = ok && kind == 1 ? p.v_scale[(int64_t)phys * p.num_kv_heads + g] : 1.0f;
    }
  }
  __syncthreads();

  // Per-lane byte offsets inside a page.
  const uint32_t krow = (uint32_t)p.num_kv_heads * D * 2u;   // bytes per token row, fp16
  const uint32_t vrow = (uint32_t)p.num_kv_heads * D;        // bytes per token row, E4M3
  const uint32_t kqoff = (uint32_t)(lane & 15) * krow + 16u * (lane >> 4);      // K: token l%16
  const uint32_t kqoff8 = (uint32_t)(lane & 15) * vrow + 8u * (lane >> 4);      // BASE K bytes
  const uint32_t voff16 = 4u * (lane >> 4) * krow + (uint32_t)(lane & 15) * (D / 8);  // V16: tokens 4(l/16)+i
  const uint32_t voff8 = 4u * (lane >> 4) * vrow + (uint32_t)(lane & 15) * (D / 16);  // V8
  const int64_t kpage = (int64_t)kPage * krow, vpage8 = (int64_t)kPage * vrow;
  bool bad = false;

  auto issue = [&](Slot<D>& sl, int pq) {
    int m;
    if constexpr (HAS_BASE) {  // no early exit: a missing page issues range-0 loads
      m = pq < pend ? __builtin_amdgcn_readfirstlane(sm.meta[pq - pbeg]) : -2;
      bad |= m == -1;
    } else {
      sl.ok = false;
      if (pq >= pend) return;
      m = __builtin_amdgcn_readfirstlane(sm.meta[pq - pbeg]);
      if (m < 0) { bad = true; return; }
    }
    sl.ok = m >= 0;
    const int phys = sl.ok ? m >> KBITS : 0;
    sl.kind = sl.ok ? m & ((1 << KBITS) - 1) : 0;
    const char* kb;
    const char* vb;
    uint32_t kbytes, vbytes;
    if (HAS_BASE && sl.kind == 2) {  // half (phys & 1) of TARGET block phys >> 1, bytes
      const int64_t off = (int64_t)(phys >> 1) * kpage + (int64_t)(phys & 1) * vpage8 + (int64_t)g * D;
      kb = reinterpret_cast<const char*>(p.k_target) + off;
      vb = reinterpret_cast<const char*>(p.v_target) + off;
      kbytes = vbytes = (uint32_t)vpage8 - (uint32_t)g * D;
    } else {
      kb = reinterpret_cast<const char*>(sl.kind ? p.k_compact : p.k_target) + phys * kpage + (int64_t)g * D * 2;
      vb = sl.kind ? reinterpret_cast<const char*>(p.v_compact) + phys * vpage8 + (int64_t)g * D
                   : reinterpret_cast<const char*>(p.v_target) + phys * kpage + (int64_t)g * D * 2;
      kbytes = (uint32_t)kpage - (uint32_t)g * D * 2;
      vbytes = sl.kind ? (uint32_t)vpage8 - (uint32_t)g * D : kbytes;
    }
    if (!sl.ok) {
      kbytes = 0u;
      vbytes = 0u;
    }
    sl.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sm.scale[pq - pbeg])));
    load_page<D, HAS_BASE, KAUX, VAUX>(sl.r, sl.kind, kb, vb, kbytes, vbytes, kqoff, kqoff8, voff16, voff8, krow, vrow);
  };
  // kSlots register page buffers: pages pg+4 .. pg+4(kSlots-1) load while page pg
  // computes.  Slots are named variables (never an indexed array) so they stay
  // in registers.
  static_assert(kSlots >= 2 && kSlots <= 6, "kSlots in 2..6");
  int pg = pbeg + wave;
  Slot<D> s0, s1, s2, s3, s4, s5;
#define EKV_STEP(CUR, NXT)                                                        \
  issue(NXT, pg + (kSlots - 1) * kWaves);                                         \
  if (CUR.ok) process_page<D, G, HAS_BASE>(st, CUR.r, p, CUR.kind, CUR.scale, pg, len, lane); \
  pg += kWaves;                                                                   \
  if (pg >= pend) break;
  issue(s0, pg);
  if (kSlots > 2) issue(s1, pg + kWaves);
  if (kSlots > 3) issue(s2, pg + 2 * kWaves);
  if (kSlots > 4) issue(s3, pg + 3 * kWaves);
  if (kSlots > 5) issue(s4, pg + 4 * kWaves);
  while (pg < pend) {
    if constexpr (kSlots == 2) {
      EKV_STEP(s0, s1) EKV_STEP(s1, s0)
    } else if constexpr (kSlots == 3) {
      EKV_STEP(s0, s2) EKV_STEP(s1, s0) EKV_STEP(s2, s1)
    } else if constexpr (kSlots == 4) {
      EKV_STEP(s0, s3) EKV_STEP(s1, s0) EKV_STEP(s2, s1) EKV_STEP(s3, s2)
    } else if constexpr (kSlots == 5) {
      EKV_STEP(s0, s4) EKV_STEP(s1, s0) EKV_STEP(s2, s1) EKV_STEP(s3, s2) EKV_STEP(s4, s3)
    } else {
      EKV_STEP(s0, s5) EKV_STEP(s1, s0) EKV_STEP(s2, s1) EKV_STEP(s3, s2) EKV_STEP(s4, s3)
      EKV_STEP(s5, s4)
    }
  }
#undef EKV_STEP

  // This wavefront's totals: head h's sum spans lanes h, h+16, h+32, h+48;
  // its output rows are acc[e][i] for h = 4(l/16)+i, d = (D/16)(l%16) + e.
  float L = st.l + shfl_xor(st.l, 16);
  L += shfl_xor(L, 32);
  if (st.aexp != 0) {  // back to true values (exact power-of-two scaling)
    const float k = as_f32((uint32_t)(st.aexp + 127) << 23);
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[e][i] *= k;
  }
  {
    const int tq = lane >> 4, dq = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * tq + i;
      if (h < G) {
#pragma unroll
        for (int e = 0; e < NE; ++e) sm.acc[wave][h][NE * dq + e] = st.acc[e][i];
      }
    }
    if (tq == 0 && dq < G) {
      sm.m[wave][dq] = st.m;
      sm.l[wave][dq] = L;
    }
  }
  if (lane == 0) sm.bad[wave] = bad ? 1 : 0;
  __syncthreads();
}

// Combines the wavefronts' results in sm into element (h, d): running max M
// (log2 units), sum L and unnormalized o; `bad` if any wavefront met a bad
// page.
template <int D, int G, int NW, class SM>
__device__ __forceinline__ void combine_waves(const SM& sm, int h, int d, float& M, float& L,
                                              float& o) {
  M = sm.m[0][h];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
  o = 0.f;
  L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float f = fast_exp2(sm.m[w][h] - M);
    o += sm.acc[w][h][d] * f;
    L += sm.l[w][h] * f;
  }
}

template <int NW, class SM>
__device__ __forceinline__ bool any_bad(const SM& sm) {
  bool bad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) bad |= sm.bad[w] != 0;
  return bad;
}

// Normalized output rows (and LSE) of the G query heads of KV head g in
// sequence b from a piece that covers the whole sequence.
template <int D, int G, int NW, class SM>
__device__ __forceinline__ void write_rows(const DecodeParams& p, const SM& sm, int b, int g) {
  const bool bad = any_bad<NW>(sm);
  const float qnan = __builtin_nanf("");
  const int64_t row0 = (int64_t)b * p.num_q_heads + g * G;
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int h = i / D, d = i % D;
    float M, L, o;
    combine_waves<D, G, NW>(sm, h, d, M, L, o);
    const float v = bad ? qnan : o * (1.0f / L);
    if (p.out_f32) static_cast<float*>(p.out)[(row0 + h) * D + d] = v;
    else static_cast<f16*>(p.out)[(row0 + h) * D + d] = (f16)v;
    if (p.lse && d == 0) p.lse[row0 + h] = bad ? qnan : (M + log2f(L)) * kLn2;
  }
}

// Partial result (unnormalized acc, max, sum) of a piece into slot `slot`
// (G records of D + 2 floats: part_acc[slot][G][D], part_ml[slot][G][2]).
template <int D, int G, int NW, class SM>
__device__ __forceinline__ void write_partial(const DecodeParams& p, const SM& sm, int64_t slot) {
  const bool bad = any_bad<NW>(sm);
  const float qnan = __builtin_nanf("");
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int h = i / D, d = i % D;
    float M, L, o;
    combine_waves<D, G, NW>(sm, h, d, M, L, o);
    p.part_acc[(slot * G + h) * D + d] = bad ? qnan : o;
    if (d == 0) {
      p.part_ml[(slot * G + h) * 2 + 0] = bad ? qnan : M;
      p.part_ml[(slot * G + h) * 2 + 1] = bad ? qnan : L;
    }
  }
}

// NW wavefronts per workgroup = (split, KV head g, sequence b).  DIRECT (one
// split per sequence, p.n_splits == 1): the workgroup normalizes its result
// and writes out / lse itself, and no merge kernel runs.
template <int D, int G, int MODE, int NW, bool DIRECT>
__global__ __launch_bounds__(NW * kWave, kMinWaves) void decode_splitk_kernel(DecodeParams p) {
  __shared__ PieceSmem<D, G, NW> sm;
  const int lane = threadIdx.x & (kWave - 1);
  // wavefront index made provably uniform, so page metadata becomes scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int split = kHeadMajorGrid ? blockIdx.y : blockIdx.x;
  const int g = kHeadMajorGrid ? blockIdx.x : blockIdx.y;
  const int b = blockIdx.z;
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npages = (len + kPage - 1) / kPage;
  const int pbeg = split * p.pages_per_split;
  if (pbeg >= npages) {  // the merge ignores splits past the sequence end
    if (DIRECT) write_empty_rows<D, G>(p, b, g);  // len 0: out 0, lse -inf
    return;
  }
  const int pend = min(pbeg + p.pages_per_split, npages);
  run_piece<D, G, MODE, NW, kKAux, kVAux>(p, sm, b, g, len, pbeg, pend, lane, wave);
  if constexpr (DIRECT) write_rows<D, G, NW>(p, sm, b, g);
  else write_partial<D, G, NW>(p, sm, ((int64_t)(b * p.num_kv_heads + g) * p.n_splits + split));
}

// ---------------------------------------------------------------------------
// Balanced plan for ragged batches.  All page-heads of the batch, in the
// order (sequence, KV head, page), are cut into n_wg equal ranges
// [r(i), r(i+1)), r(i) = floor(i W / n_wg), one per workgroup, in one round.
// A workgroup walks its range piece by piece (a piece = the part of one
// (sequence, KV head) inside the range): a piece that is a whole (sequence,
// KV head) is written as output directly; a piece cut by the range ends is a
// partial result in the workgroup's slot 0 (the piece at the start of the
// range) or slot 1 (the piece at its end).  The merge kernel then combines,
// for each cut (sequence, KV head), the tail piece of its first workgroup and
// the head pieces of the following ones.

__device__ __forceinline__ int seq_pages(const DecodeParams& p, int b) {
  return (min(max(p.seq_lens[b], 0), p.max_seq_len) + kPage - 1) / kPage;
}

// Workgroup whose range holds flattened position x.
__device__ __forceinline__ int wg_of(int64_t x, int64_t W, int n) { return (int)(((x + 1) * n - 1) / W); }
__device__ __forceinline__ int64_t wg_start(int i, int64_t W, int n) { return (int64_t)i * W / n; }

template <int D, int G, int MODE>
__global__ __launch_bounds__(kBalancedWaves * kWave, kMinWaves) void decode_balanced_kernel(DecodeParams p) {
  constexpr int NW = kBalancedWaves;
  __shared__ PieceSmem<D, G, NW, kBalancedMaxPages> sm;
  __shared__ int s_pref[kDecodeMaxBalancedBatch + 1];  // exclusive prefix sums of page counts
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int B = p.batch;
  if (wave == 0) {  // one wavefront scans the page counts
    const int per = (B + kWave - 1) / kWave;
    const int lo = lane * per, hi = min(B, lo + per);
    int sum = 0;
    for (int b = lo; b < hi; ++b) sum += seq_pages(p, b);
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += t;
    }
    int run = incl - sum;
    for (int b = lo; b < hi; ++b) {
      s_pref[b] = run;
      run += seq_pages(p, b);
    }
    if (lane == kWave - 1) s_pref[B] = incl;
  }
  __syncthreads();
  const int H = p.num_kv_heads;
  const int64_t W = (int64_t)H * s_pref[B];
  const int n = p.n_wg, i = blockIdx.x;
  const int64_t w0 = wg_start(i, W, n), w1 = wg_start(i + 1, W, n);
  if (w0 == w1) {  // empty range (fewer page-heads than workgroups): a neutral head record,
    // since the merge reads the head slots of every workgroup a cut sequence spans
    for (int e = threadIdx.x; e < G * D; e += NW * kWave) {
      p.part_acc[2 * (int64_t)i * G * D + e] = 0.f;
      if (e < G) {
        p.part_ml[(2 * (int64_t)i * G + e) * 2 + 0] = kNegBig;
        p.part_ml[(2 * (int64_t)i * G + e) * 2 + 1] = 0.f;
      }
    }
    return;
  }
  int64_t q = w0;
  while (q < w1) {
    // sequence of position q: the last b with H * pref[b] <= q (skips empty ones)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)H * s_pref[mid] <= q) lo = mid;
      else hi = mid - 1;
    }
    const int b = lo;
    const int np = s_pref[b + 1] - s_pref[b];
    const int64_t off = q - (int64_t)H * s_pref[b];
    const int g = (int)(off / np);
    const int page = (int)(off - (int64_t)g * np);
    const int64_t seg = (int64_t)H * s_pref[b] + (int64_t)g * np;
    const int pend = (int)(min(w1, seg + np) - seg);
    const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
    run_piece<D, G, MODE, NW, kKAux, kVAux>(p, sm, b, g, len, page, pend, lane, wave);
    if (page == 0 && pend == np) write_rows<D, G, NW>(p, sm, b, g);
    else write_partial<D, G, NW>(p, sm, 2 * (int64_t)i + (q == w0 ? 0 : 1));
    q = seg + pend;
    __syncthreads();  // sm is reused by the next piece
  }
}

// One wavefront per (query head, sequence): combine the partial results.
// Split plan: splits 0 .. nsplit-1 of the sequence.  Balanced plan: the
// pieces of the workgroups whose ranges cut this (sequence, KV head); a
// (sequence, KV head) inside one range was written by its workgroup.
template <int D, bool BALANCED>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeParams p) {
  constexpr int PER = D / kWave;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = h / G, hh = h - g * G;
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npages = (len + kPage - 1) / kPage;
  const int64_t row = (int64_t)b * p.num_q_heads + h;

  int nsplit;
  int64_t slot0 = 0, first = 0;  // record of piece s: s == 0 ? first : slot0 + 2 s
  if constexpr (BALANCED) {
    int before = 0, total = 0;
    for (int x = lane; x < p.batch; x += kWave) {
      const int n = seq_pages(p, x);
      total += n;
      before += x < b ? n : 0;
    }
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) {
      total += __shfl_xor(total, x, kWave);
      before += __shfl_xor(before, x, kWave);
    }
    if (npages == 0) {
      nsplit = 0;
    } else {
      const int64_t W = (int64_t)p.num_kv_heads * total;
      const int64_t start = (int64_t)p.num_kv_heads * before + (int64_t)g * npages;
      const int i0 = wg_of(start, W, p.n_wg), i1 = wg_of(start + npages - 1, W, p.n_wg);
      if (i0 == i1) return;  // written by its workgroup
      nsplit = i1 - i0 + 1;
      first = 2 * (int64_t)i0 + (start == wg_start(i0, W, p.n_wg) ? 0 : 1);
      slot0 = 2 * (int64_t)i0;  // piece s >= 1: head slot of workgroup i0 + s
    }
  } else {
    nsplit = (npages + p.pages_per_split - 1) / p.pages_per_split;
    first = (int64_t)(b * p.num_kv_heads + g) * p.n_splits;
    slot0 = first;
  }
  auto rec = [&](int s) -> int64_t {
    const int64_t slot = BALANCED ? (s == 0 ? first : slot0 + 2 * (int64_t)s) : slot0 + s;
    return slot * G + hh;
  };

  float o[PER];
  float lse_v;
  if (nsplit == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    lse_v = -__builtin_inff();
  } else {
    // split statistics are spread over the lanes (split s in lane s % 64), so
    // their loads and the max / sum reductions run in parallel
    float M = kNegBig;
    bool bad = false;
    for (int s0 = 0; s0 < nsplit; s0 += kWave) {
      const int s = s0 + lane;
      const float ms = s < nsplit ? p.part_ml[rec(s) * 2] : kNegBig;
      bad |= ms != ms;
      M = fmaxf(M, ms);
    }
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) M = fmaxf(M, shfl_xor(M, x));
    bad = __ballot(bad) != 0;
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kWave) {
      const int s = s0 + lane;
      float f_lane = 0.f;
      if (s < nsplit) {
        const int64_t k = rec(s);
        f_lane = fast_exp2(p.part_ml[k * 2] - M);
        L += p.part_ml[k * 2 + 1] * f_lane;
      }
      const int cnt = min(kWave, nsplit - s0);
      for (int j = 0; j < cnt; ++j) {
        const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f_lane), j));
        const int64_t k = rec(s0 + j);
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += p.part_acc[k * D + lane + kWave * i] * f;
      }
    }
#pragma unroll
    for (int x = 1; x < kWave; x <<= 1) L += shfl_xor(L, x);
    const float inv = 1.0f / L;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] *= inv;
    lse_v = (M + log2f(L)) * kLn2;
    if (bad) {
      const float qnan = __builtin_nanf("");
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] = qnan;
      lse_v = qnan;
    }
  }
  if (p.out_f32) {
    float* out = static_cast<float*>(p.out) + row * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + kWave * i] = o[i];
  } else {
    f16* out = static_cast<f16*>(p.out) + row * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + kWave * i] = (f16)o[i];
  }
  if (p.lse && lane == 0) p.lse[row] = lse_v;
}

template <int D, int G, int NW, bool DIRECT>
hipError_t launch_split(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  const int mode = p.has_base ? (p.fidelity ? 2 : 3) : (p.fidelity ? 1 : 0);
  const dim3 block(NW * kWave);
  switch (mode) {
    case 0: hipLaunchKernelGGL((decode_splitk_kernel<D, G, 0, NW, DIRECT>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((decode_splitk_kernel<D, G, 1, NW, DIRECT>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_splitk_kernel<D, G, 2, NW, DIRECT>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_splitk_kernel<D, G, 3, NW, DIRECT>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_balanced(const DecodeParams& p, hipStream_t stream) {
  const int mode = p.has_base ? (p.fidelity ? 2 : 3) : (p.fidelity ? 1 : 0);
  const dim3 grid(p.n_wg), block(kBalancedWaves * kWave);
  switch (mode) {
    case 0: hipLaunchKernelGGL((decode_balanced_kernel<D, G, 0>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((decode_balanced_kernel<D, G, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_balanced_kernel<D, G, 2>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_balanced_kernel<D, G, 3>), grid, block, 0, stream, p); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, true>), dim3(p.num_q_heads, p.batch), dim3(kWave), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, hipStream_t stream) {
  if (p.n_wg > 0) return launch_balanced<D, G>(p, stream);
  const dim3 grid = kHeadMajorGrid ? dim3(p.num_kv_heads, p.n_splits, p.batch)
                                   : dim3(p.n_splits, p.num_kv_heads, p.batch);
  if (p.n_splits == 1) {
    // One split per sequence: the split kernel writes the output.  Up to 256
    // (sequence, KV head) groups, 8 wavefronts per group keep 2 per SIMD.
    return (int64_t)p.batch * p.num_kv_heads <= 256 ? launch_split<D, G, 8, true>(p, grid, stream)
                                                     : launch_split<D, G, 4, true>(p, grid, stream);
  }
  if (p.n_splits > 0) {
    const hipError_t e = launch_split<D, G, 4, false>(p, grid, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_merge_kernel<D, false>), dim3(p.num_q_heads, p.batch), dim3(kWave), 0, stream,
                     p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: return launch_dg<D, 1>(p, stream);
    case 2: return launch_dg<D, 2>(p, stream);
    case 4: return launch_dg<D, 4>(p, stream);
    case 8: return launch_dg<D, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int32_t decode_auto_pages_per_split(int32_t batch, int32_t num_kv_heads, int32_t max_pages) {
  // About 512 workgroups (two 4-wavefront groups per CU) if every sequence had
  // max_pages pages: measured best on the 256-CU part; splits are whole
  // multiples of the 4 wavefronts' page stride, between 16 and 512 pages.
  if (max_pages <= 0) return 16;
  const int64_t seqs = (int64_t)batch * num_kv_heads;
  // 192..256 (sequence, KV head) groups: one split each in 8-wavefront
  // workgroups fills the chip as well as two 4-wavefront splits would, and
  // the split kernel writes the output itself (no partials, no merge launch).
  if (seqs >= 192 && seqs <= 256 && max_pages <= kMaxSplitPages) return max_pages < 16 ? 16 : max_pages;
  int64_t c = (seqs * max_pages + 511) / 512;
  c = (c + 3) / 4 * 4;
  return (int32_t)(c < 16 ? 16 : (c > 512 ? 512 : c));
}

size_t decode_scratch_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t n_splits) {
  (void)num_kv_heads;
  if (n_splits <= 1) return 0;  // one split writes the output directly
  const size_t rows = (size_t)batch * num_q_heads * (size_t)n_splits;  // (b, g, split, hh)
  const size_t acc = rows * head_dim * sizeof(float);
  const size_t acc_aligned = (acc + 255) & ~(size_t)255;
  return acc_aligned + rows * 2 * sizeof(float);
}

int32_t decode_balanced_workgroups(int32_t batch, int32_t num_kv_heads, int32_t max_pages) {
  // one round: one 8-wavefront workgroup per CU on the 256-CU part (2
  // wavefronts per SIMD; measured 1% ahead of two 4-wavefront workgroups
  // per CU), more (whole rounds) when a range would exceed the LDS
  // page-metadata stage
  const int64_t work = (int64_t)batch * num_kv_heads * max_pages;
  int64_t n = kBalancedRound;
  while ((work + n - 1) / n > kBalancedMaxPages) n += kBalancedRound;
  return (int32_t)n;
}

size_t decode_balanced_scratch_bytes(int32_t n_wg, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim) {
  const size_t recs = (size_t)n_wg * 2 * (num_q_heads / num_kv_heads);
  const size_t acc = (recs * head_dim * sizeof(float) + 255) & ~(size_t)255;
  return acc + recs * 2 * sizeof(float);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (p.head_dim == 64) return launch_d<64>(p, stream);
  if (p.head_dim == 128) return launch_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace ekv

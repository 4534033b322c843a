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
//   workgroup = (split of C pages, KV head g, sequence b); 4 wavefronts take
//   the split's pages round-robin.  Inside a wavefront a page is 16 tokens x
//   D: lane = (token pair tp = lane/8 -> tokens tp, tp+8; d-octet j = lane%8).
//   Lane j owns d in {64c + 8j + e : c < D/64, e < 8}, so each 16-byte load
//   instruction covers 8 token rows x 128 contiguous bytes.
//   QK^T: v_dot2_f32_f16 over the lane's d (fp32 accumulate), then a 3-step
//   DPP sum across the octet.  The G = Hq/Hkv query heads of the group share
//   every K/V load.
//   Softmax: online, per token-pair group (8 groups per wavefront), in log2
//   units; the running max is raised only when a page max exceeds it by more
//   than kTau (exact: softmax is shift invariant; it only skips rescales).
//   PV: fp32 p times the fp16 value, fp32 accumulate (v_fma_mix_f32).
//   Compact pages expand their E4M3 bytes in registers with the gfx950
//   scaled conversion by the power-of-two part 2^e of the page-head scale
//   (exact: code * 2^e is an fp16 value); the mantissa part f of the scale
//   multiplies p in fp32.  Both kinds meet in one fp16-value PV path.  The flag is per page, so the
//   branch is wavefront-uniform.
//   End of split: groups merge by shuffles, wavefronts through LDS; the split
//   writes (max, sum, unnormalized acc) partials.  The merge kernel combines
//   splits: M = max m_s, L = sum l_s 2^(m_s-M), o = sum acc_s 2^(m_s-M) / L,
//   lse = (M + log2 L) ln 2.
#include "ekv_device.hpp"
#include "ekv_internal.hpp"

namespace ekv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kTau = 8.0f;          // deferred-rescale threshold (log2 units)
constexpr float kNegBig = -1.0e30f;   // "no token yet" running max
constexpr bool kHeadMajorGrid = true; // launch order: the KV heads of one (sequence, split) adjacent
constexpr int kMaxSplitPages = 512;   // pages per split (metadata staged in LDS)

template <int D>
struct PageRegs {
  f16x8 k[D / 32];        // K[token lane%16][32kb + 8(lane/16) .. +8]: MFMA B operand per kb
  uint32_t v[2][D / 16];  // V rows of tokens tp, tp+8 at this lane's d-set (TARGET fp16;
                          // COMPACT: the first D/32 dwords hold D/8 E4M3 bytes)
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
// descriptors (wavefront-uniform, SGPRs) cover exactly one page of one KV head,
// so the hardware range check keeps every access inside that page; `koff`/
// `voff` are per-lane 32-bit byte offsets (token tp, d-octet j) and the
// second token's 8-row stride goes in the scalar offset.
template <int D>
__device__ __forceinline__ void load_page(PageRegs<D>& r, int kind, const char* kbase,
                                          const char* vbase, uint32_t kbytes, uint32_t vbytes,
                                          uint32_t kqoff, uint32_t koff, uint32_t voff,
                                          uint32_t krow8, uint32_t vrow8) {
  constexpr int NC = D / 64;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, kbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, vbytes, kBufferFlags);
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    r.k[kb] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, kqoff + 64u * kb, 0, 0));
  if (kind == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(vr, koff + 128u * c, t * krow8, 0);
        r.v[t][4 * c + 0] = y.x; r.v[t][4 * c + 1] = y.y;
        r.v[t][4 * c + 2] = y.z; r.v[t][4 * c + 3] = y.w;
      }
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(vr, voff + 64u * c, t * vrow8, 0);
        r.v[t][2 * c + 0] = y.x; r.v[t][2 * c + 1] = y.y;
      }
    // keep every element of the register array defined on both paths (no scratch)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int w = D / 32; w < D / 16; ++w) r.v[t][w] = 0u;
  }
}

template <int D, int G>
struct State {
  f16x8 qa[D / 32];  // Q[head lane%16][32kb + 8(lane/16) .. +8]: MFMA A operand (0 for head >= G)
  float m[G], l[G];
  float acc[G][D / 8];
};

template <int D, int G>
__device__ __forceinline__ void process_page(State<D, G>& st, PageRegs<D>& r, const DecodeParams& p,
                                             int kind, float scale, int pg, int len, int tp) {
  constexpr int DW = D / 16;
  // Compact scale s = 2^e * f, f in [1, 2): the conversion applies the exact power of two,
  // p carries f.  (Scales are positive normal fp32 values.)
  const uint32_t sbits = kind ? __builtin_bit_cast(uint32_t, scale) : 0x3F800000u;
  const float s_pow2 = as_f32(sbits & 0x7F800000u);
  const float s_frac = as_f32((sbits & 0x807FFFFFu) | 0x3F800000u);
  const int t0 = pg * kPage + tp;
  const bool ok0 = t0 < len, ok1 = t0 + 8 < len;
  const bool partial = pg * kPage + kPage > len;  // wavefront-uniform

  // S[h][t] = Q . K^T on the matrix cores: rows = heads (padded to 16), columns = the
  // page's 16 tokens; lane l receives S[4(l/16)+i][l%16], i < 4.
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.qa[kb], r.k[kb], sacc, 0, 0, 0);
  // Move the scores of tokens tp and tp+8 to this lane (PV layout).
  float s0[G], s1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int src = 16 * (h / 4);
    const float v = sacc[h % 4];
    s0[h] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (src + tp), __builtin_bit_cast(int, v))) * p.scale_log2;
    s1[h] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (src + tp + 8), __builtin_bit_cast(int, v))) * p.scale_log2;
  }
  if (partial) {  // last page of the sequence: drop slots >= len (their contents are undefined)
    const float ninf = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s0[h] = ok0 ? s0[h] : ninf;
      s1[h] = ok1 ? s1[h] : ninf;
    }
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      r.v[0][w] = ok0 ? r.v[0][w] : 0u;
      r.v[1][w] = ok1 ? r.v[1][w] : 0u;
    }
  }

  bool raise = false;
  float mnew[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = fmaxf(s0[h], s1[h]);
    mnew[h] = (mx > st.m[h] + kTau) ? mx : st.m[h];
    raise |= mnew[h] != st.m[h];
  }
  if (__ballot(raise)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = fast_exp2(st.m[h] - mnew[h]);  // 1 when unchanged, 0 from kNegBig
      st.l[h] *= a;
#pragma unroll
      for (int e = 0; e < D / 8; ++e) st.acc[h][e] *= a;
      st.m[h] = mnew[h];
    }
  }

  float pf[G][2];  // fp32 probabilities of the lane's two tokens (times f on compact pages)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p0 = fast_exp2(s0[h] - st.m[h]);
    const float p1 = fast_exp2(s1[h] - st.m[h]);
    st.l[h] += p0 + p1;
    pf[h][0] = p0 * s_frac;
    pf[h][1] = p1 * s_frac;
  }

  // PV with fp32 p and fp32 accumulation; the fp16 value operand is exact
  // (v_fma_mix_f32 reads either half of a packed fp16 register).
  if (kind == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int w = 0; w < DW; ++w) {
        const f16x2 v = as_f16x2(r.v[t][w]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          st.acc[h][2 * w] = __builtin_fmaf((float)v.x, pf[h][t], st.acc[h][2 * w]);
          st.acc[h][2 * w + 1] = __builtin_fmaf((float)v.y, pf[h][t], st.acc[h][2 * w + 1]);
        }
      }
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int w = 0; w < DW / 2; ++w) {
        const f16x2 lo = e4m3x2_scaled_f16(r.v[t][w], s_pow2, false);  // d = 4w, 4w+1
        const f16x2 hi = e4m3x2_scaled_f16(r.v[t][w], s_pow2, true);   // d = 4w+2, 4w+3
#pragma unroll
        for (int h = 0; h < G; ++h) {
          st.acc[h][4 * w + 0] = __builtin_fmaf((float)lo.x, pf[h][t], st.acc[h][4 * w + 0]);
          st.acc[h][4 * w + 1] = __builtin_fmaf((float)lo.y, pf[h][t], st.acc[h][4 * w + 1]);
          st.acc[h][4 * w + 2] = __builtin_fmaf((float)hi.x, pf[h][t], st.acc[h][4 * w + 2]);
          st.acc[h][4 * w + 3] = __builtin_fmaf((float)hi.y, pf[h][t], st.acc[h][4 * w + 3]);
        }
      }
  }
}

template <int D, int G, bool FLAGS>
__global__ __launch_bounds__(kThreads, (G * D >= 1024 ? 1 : 2)) void decode_splitk_kernel(DecodeParams p) {
  constexpr int NC = D / 64;
  constexpr int DE = D / 8;
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_bad[kWaves];
  __shared__ int s_meta[kMaxSplitPages];

  const int lane = threadIdx.x & (kWave - 1);
  // wavefront index made provably uniform, so page metadata becomes scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int j = lane & 7, tp = lane >> 3;
  const int split = kHeadMajorGrid ? blockIdx.y : blockIdx.x;
  const int g = kHeadMajorGrid ? blockIdx.x : blockIdx.y;
  const int b = blockIdx.z;
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npages = (len + kPage - 1) / kPage;
  const int pbeg = split * p.pages_per_split;
  if (pbeg >= npages) return;  // the merge ignores splits past the sequence end
  const int pend = min(pbeg + p.pages_per_split, npages);

  State<D, G> st;
  {
    const int qh = lane & 15, qc = lane >> 4;
    const uint16_t* qp = p.q + ((int64_t)b * p.num_q_heads + g * G + qh) * D + 8 * qc;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      st.qa[kb] = qh < G ? __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(qp + 32 * kb)) : f16x8{};
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegBig;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DE; ++e) st.acc[h][e] = 0.f;
  }

  // Stage this split's page metadata in LDS once: (phys << 1 | kind), or -1
  // for an out-of-range id or unknown flag.  Per-page reads are then LDS
  // reads, which never wait on the vector-memory counter of in-flight pages.
  {
    const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride;
    const uint8_t* fl = FLAGS ? p.fidelity + (int64_t)b * p.pt_stride : nullptr;
    for (int i = threadIdx.x; i < pend - pbeg; i += kThreads) {
      const int phys = pt[pbeg + i];
      const int kind = FLAGS ? (int)fl[pbeg + i] : p.uniform_kind;
      const bool ok = (kind == 0 && (unsigned)phys < (unsigned)p.n_target) ||
                      (kind == 1 && (unsigned)phys < (unsigned)p.n_compact);
      s_meta[i] = ok ? (phys << 1) | kind : -1;
    }
  }
  __syncthreads();

  // Per-lane byte offsets inside a page (token tp, d-octet j) and 8-row strides.
  const uint32_t krow = (uint32_t)p.num_kv_heads * D * 2u;   // bytes per token row, fp16
  const uint32_t vrow = (uint32_t)p.num_kv_heads * D;        // bytes per token row, E4M3
  const uint32_t koff = (uint32_t)tp * krow + 16u * j;          // V16 rows (PV layout)
  const uint32_t kqoff = (uint32_t)(lane & 15) * krow + 16u * (lane >> 4);  // K rows (MFMA layout)
  const uint32_t voff = (uint32_t)tp * vrow + 8u * j;
  const int64_t kpage = (int64_t)kPage * krow, vpage8 = (int64_t)kPage * vrow;
  bool bad = false;

  auto issue = [&](Slot<D>& sl, int pq) {
    sl.ok = false;
    if (pq >= pend) return;
    const int m = __builtin_amdgcn_readfirstlane(s_meta[pq - pbeg]);
    if (m < 0) { bad = true; return; }
    const int phys = m >> 1;
    sl.kind = m & 1;
    sl.ok = true;
    const char* kb = reinterpret_cast<const char*>(sl.kind ? p.k_compact : p.k_target) +
                     phys * kpage + (int64_t)g * D * 2;
    const char* vb = sl.kind ? reinterpret_cast<const char*>(p.v_compact) + phys * vpage8 + (int64_t)g * D
                             : reinterpret_cast<const char*>(p.v_target) + phys * kpage + (int64_t)g * D * 2;
    const uint32_t kbytes = (uint32_t)kpage - (uint32_t)g * D * 2;
    const uint32_t vbytes = sl.kind ? (uint32_t)vpage8 - (uint32_t)g * D : kbytes;
    sl.scale = sl.kind ? p.v_scale[(int64_t)phys * p.num_kv_heads + g] : 1.0f;
    load_page<D>(sl.r, sl.kind, kb, vb, kbytes, vbytes, kqoff, koff, voff, 8u * krow, 8u * vrow);
  };
  // Two slots: page pg+4 loads while page pg computes.
  Slot<D> sa, sb;
  int pg = pbeg + wave;
  issue(sa, pg);
  while (pg < pend) {
    issue(sb, pg + kWaves);
    if (sa.ok) process_page<D, G>(st, sa.r, p, sa.kind, sa.scale, pg, len, tp);
    pg += kWaves;
    if (pg >= pend) break;
    issue(sa, pg + kWaves);
    if (sb.ok) process_page<D, G>(st, sb.r, p, sb.kind, sb.scale, pg, len, tp);
    pg += kWaves;
  }

  // Merge the 8 token-pair groups of this wavefront (lanes with equal j).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = st.m[h];
    M = fmaxf(M, dpp<kDppRowRor8>(M));
    M = fmaxf(M, shfl_xor(M, 16));
    M = fmaxf(M, shfl_xor(M, 32));
    const float f = fast_exp2(st.m[h] - M);
    float L = st.l[h] * f;
    L += dpp<kDppRowRor8>(L);
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
#pragma unroll
    for (int e = 0; e < DE; ++e) {
      float a = st.acc[h][e] * f;
      a += dpp<kDppRowRor8>(a);
      a += shfl_xor(a, 16);
      a += shfl_xor(a, 32);
      st.acc[h][e] = a;
    }
    st.m[h] = M;
    st.l[h] = L;
  }
  if (tp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DE; ++e) s_acc[wave][h][64 * (e / 8) + 8 * j + (e % 8)] = st.acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = st.m[h];
      s_l[wave][h] = st.l[h];
    }
    s_bad[wave] = bad ? 1 : 0;
  }
  __syncthreads();

  // Merge the wavefronts and write this split's partial result.
  const bool anybad = (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) != 0;
  const float qnan = __builtin_nanf("");
  const int64_t slot = ((int64_t)(b * p.num_kv_heads + g) * p.n_splits + split) * G;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += s_acc[w][h][d] * fast_exp2(s_m[w][h] - M);
    p.part_acc[(slot + h) * D + d] = anybad ? qnan : o;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += s_l[w][h] * fast_exp2(s_m[w][h] - M);
    p.part_ml[(slot + h) * 2 + 0] = anybad ? qnan : M;
    p.part_ml[(slot + h) * 2 + 1] = anybad ? qnan : L;
  }
}

// One wavefront per (query head, sequence): combine the splits.
template <int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeParams p) {
  constexpr int PER = D / kWave;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = h / G, hh = h - g * G;
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npages = (len + kPage - 1) / kPage;
  const int nsplit = (npages + p.pages_per_split - 1) / p.pages_per_split;
  const int64_t row = (int64_t)b * p.num_q_heads + h;

  float o[PER];
  float lse_v;
  if (nsplit == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    lse_v = -__builtin_inff();
  } else {
    const int64_t base = (int64_t)(b * p.num_kv_heads + g) * p.n_splits;
    float M = kNegBig;
    bool bad = false;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = p.part_ml[((base + s) * G + hh) * 2];
      bad |= ms != ms;
      M = fmaxf(M, ms);
    }
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const int64_t k = (base + s) * G + hh;
      const float f = fast_exp2(p.part_ml[k * 2] - M);
      L += p.part_ml[k * 2 + 1] * f;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += p.part_acc[k * D + lane + kWave * i] * f;
    }
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

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid = kHeadMajorGrid ? dim3(p.num_kv_heads, p.n_splits, p.batch)
                                   : dim3(p.n_splits, p.num_kv_heads, p.batch);
  if (p.n_splits > 0) {
    if (p.fidelity)
      hipLaunchKernelGGL((decode_splitk_kernel<D, G, true>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_splitk_kernel<D, G, false>), grid, dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.num_q_heads, p.batch), dim3(kWave), 0, stream,
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
  if (max_pages <= 0) return 16;
  const int64_t seqs = (int64_t)batch * num_kv_heads;
  int32_t c = 512;
  while (c > 16 && seqs * ((max_pages + c - 1) / c) < 2048) c /= 2;
  return c;
}

size_t decode_scratch_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t n_splits) {
  (void)num_kv_heads;
  const size_t rows = (size_t)batch * num_q_heads * (size_t)n_splits;  // (b, g, split, hh)
  const size_t acc = rows * head_dim * sizeof(float);
  const size_t acc_aligned = (acc + 255) & ~(size_t)255;
  return acc_aligned + rows * 2 * sizeof(float);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (p.head_dim == 64) return launch_d<64>(p, stream);
  if (p.head_dim == 128) return launch_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace ekv

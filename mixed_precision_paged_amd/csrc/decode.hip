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

template <int D>
struct PageRegs {
  uint32_t k[2][D / 16];  // two tokens x (D/8 fp16) of this lane's d-set
  uint32_t v[2][D / 16];  // TARGET: same as k; COMPACT: first D/32 dwords hold D/8 E4M3 bytes
};

template <int D>
__device__ __forceinline__ void load_page(PageRegs<D>& r, const DecodeParams& p, int kind,
                                          int phys, int g, int tp, int j) {
  constexpr int NC = D / 64;
  const int64_t row = (int64_t)p.num_kv_heads * D;  // elements per token row of a page
  const int64_t base = (int64_t)phys * kPage * row + (int64_t)g * D;
  const uint16_t* kp = (kind ? p.k_compact : p.k_target) + base;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t off = (int64_t)(tp + 8 * t) * row + 8 * j;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 x = *reinterpret_cast<const uint4*>(kp + off + 64 * c);
      r.k[t][4 * c + 0] = x.x; r.k[t][4 * c + 1] = x.y;
      r.k[t][4 * c + 2] = x.z; r.k[t][4 * c + 3] = x.w;
    }
  }
  if (kind == 0) {
    const uint16_t* vp = p.v_target + base;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t off = (int64_t)(tp + 8 * t) * row + 8 * j;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 x = *reinterpret_cast<const uint4*>(vp + off + 64 * c);
        r.v[t][4 * c + 0] = x.x; r.v[t][4 * c + 1] = x.y;
        r.v[t][4 * c + 2] = x.z; r.v[t][4 * c + 3] = x.w;
      }
    }
  } else {
    const uint8_t* vp = p.v_compact + base;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t off = (int64_t)(tp + 8 * t) * row + 8 * j;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint2 x = *reinterpret_cast<const uint2*>(vp + off + 64 * c);
        r.v[t][2 * c + 0] = x.x; r.v[t][2 * c + 1] = x.y;
      }
    }
  }
}

template <int D, int G>
struct State {
  uint32_t q[G][D / 16];   // fp16 pairs of the lane's d-set, per query head of the group
  float m[G], l[G];
  float acc[G][D / 8];
};

template <int D, int G>
__device__ __forceinline__ void process_page(State<D, G>& st, PageRegs<D>& r, const DecodeParams& p,
                                             int kind, int phys, int g, int pg, int len, int tp) {
  constexpr int DW = D / 16;
  // Compact scale s = 2^e * f, f in [1, 2): the conversion applies the exact power of two,
  // p carries f.  (Scales are positive normal fp32 values.)
  const uint32_t sbits = kind ? __builtin_bit_cast(uint32_t, p.v_scale[(int64_t)phys * p.num_kv_heads + g])
                              : 0x3F800000u;
  const float s_pow2 = as_f32(sbits & 0x7F800000u);
  const float s_frac = as_f32((sbits & 0x807FFFFFu) | 0x3F800000u);
  const int t0 = pg * kPage + tp;
  const bool ok0 = t0 < len, ok1 = t0 + 8 < len;
  const bool partial = pg * kPage + kPage > len;  // wavefront-uniform

  float s0[G], s1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      a0 = dot2(st.q[h][w], r.k[0][w], a0);
      a1 = dot2(st.q[h][w], r.k[1][w], a1);
    }
    s0[h] = octet_sum(a0) * p.scale_log2;
    s1[h] = octet_sum(a1) * p.scale_log2;
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

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = lane & 7, tp = lane >> 3;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int npages = (len + kPage - 1) / kPage;
  const int pbeg = split * p.pages_per_split;
  if (pbeg >= npages) return;  // the merge ignores splits past the sequence end
  const int pend = min(pbeg + p.pages_per_split, npages);

  State<D, G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qp = p.q + ((int64_t)b * p.num_q_heads + g * G + h) * D + 8 * j;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 x = *reinterpret_cast<const uint4*>(qp + 64 * c);
      st.q[h][4 * c + 0] = x.x; st.q[h][4 * c + 1] = x.y;
      st.q[h][4 * c + 2] = x.z; st.q[h][4 * c + 3] = x.w;
    }
    st.m[h] = kNegBig;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DE; ++e) st.acc[h][e] = 0.f;
  }

  const int32_t* pt = p.page_table + (int64_t)b * p.pt_stride;
  const uint8_t* fl = FLAGS ? p.fidelity + (int64_t)b * p.pt_stride : nullptr;
  bool bad = false;

  auto meta = [&](int pg, int& kind, int& phys) -> bool {
    phys = pt[pg];
    kind = FLAGS ? (int)fl[pg] : p.uniform_kind;
    if (kind == 0) return (unsigned)phys < (unsigned)p.n_target;
    if (kind == 1) return (unsigned)phys < (unsigned)p.n_compact;
    return false;
  };

  // Two register buffers: the next page loads while the current one computes.
  PageRegs<D> ra, rb;
  int ka = 0, pa = 0, kb = 0, pb = 0;
  bool oka = false, okb = false;
  int pg = pbeg + wave;
  if (pg < pend) {
    oka = meta(pg, ka, pa);
    if (oka) load_page<D>(ra, p, ka, pa, g, tp, j);
  }
  while (pg < pend) {
    int pn = pg + kWaves;
    if (pn < pend) {
      okb = meta(pn, kb, pb);
      if (okb) load_page<D>(rb, p, kb, pb, g, tp, j);
    }
    if (oka) process_page<D, G>(st, ra, p, ka, pa, g, pg, len, tp);
    else bad = true;
    pg = pn;
    if (pg >= pend) break;
    pn = pg + kWaves;
    if (pn < pend) {
      oka = meta(pn, ka, pa);
      if (oka) load_page<D>(ra, p, ka, pa, g, tp, j);
    }
    if (okb) process_page<D, G>(st, rb, p, kb, pb, g, pg, len, tp);
    else bad = true;
    pg = pn;
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
  const dim3 grid(p.n_splits, p.num_kv_heads, p.batch);
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

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
// (v_mfma_f32_32x32x16_f16, gfx950).  Workgroup = 128 query rows of one
// query head of one prompt; wavefront w owns rows [32w, 32w+32).  Per 64-key
// tile the workgroup stages K (row-major) and V^T (transposed on the way in)
// in LDS, then each wavefront computes
//     S^T[key][q] = K . Q^T      (A = K from LDS, B = Q in registers)
//     O^T[d][q]  += V^T . P^T    (A = V^T from LDS, B = P^T in registers)
// so that with the 32x32 output layout every per-query quantity (running max,
// sum, rescale factor) lives in the lane whose column is that query: lane l
// holds column l%32 and half of its rows; a single xor-32 exchange completes a
// column reduction.  The key order inside the P.V contraction follows the
// S^T register layout, and V^T is read in the same order.
// Launch order: workgroups are mapped so that each XCD (8 per MI355X, each
// with its own L2) walks a contiguous range of (prompt, head, row tile), so
// the K/V rows a head reuses stay in one L2; within a head the longest
// (last) causal row tiles start first.
#include "ekv_device.hpp"
#include "ekv_internal.hpp"

namespace ekv {
namespace {

constexpr int kM = 128;        // query rows per workgroup
constexpr int kN = 64;         // keys per tile
constexpr int kThreads = 256;
constexpr float kTau = 8.0f;
constexpr float kNegBig = -1.0e30f;
constexpr int kXcds = 8;

template <int D>
struct Smem {
  static constexpr int kStride = D + 8;    // K row stride (halves): 16 B pad
  static constexpr int vStride = kN + 4;   // V^T row stride (halves): 8 B pad
  f16 k[kN * kStride];
  f16 vt[D * vStride];
};

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <int D>
struct TileRegs {
  static constexpr int KCH = kN * D / 8 / kThreads;  // 16-byte K chunks per thread
  uint4 k[KCH];
  uint4 v[4];  // 4 key rows x 8 d of one (key quad, d octet) unit
};

// Tile loads are buffer loads through per-prompt descriptors (SGPRs) whose
// range ends at the prompt's last key row of this KV head, so rows past the
// prompt read as zeros (no per-load branch).  Per-lane byte offsets are fixed
// for the whole loop; the tile's first row goes in the scalar offset.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, __amdgpu_buffer_rsrc_t kr,
                                          __amdgpu_buffer_rsrc_t vr, const uint32_t* koff,
                                          const uint32_t* voff, uint32_t tile_off) {
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KCH; ++i) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[i], tile_off, 0);
    r.k[i] = make_uint4(x.x, x.y, x.z, x.w);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[i], tile_off, 0);
    r.v[i] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(Smem<D>& s, const TileRegs<D>& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KCH; ++i) {
    const int idx = t + kThreads * i;
    const int key = idx / (D / 8), ch = idx % (D / 8);
    *reinterpret_cast<uint4*>(&s.k[key * Smem<D>::kStride + 8 * ch]) = r.k[i];
  }
  constexpr int units = (kN / 4) * (D / 8);
  if (t < units) {
    const int kq = t % (kN / 4), oc = t / (kN / 4);
    const uint32_t r0[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
    const uint32_t r1[4] = {r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
    const uint32_t r2[4] = {r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w};
    const uint32_t r3[4] = {r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // d = 8*oc + 2w and 2w+1: four keys' values, key order 4kq..4kq+3
      const uint2 even = make_uint2(perm(r1[w], r0[w], 0x05040100u), perm(r3[w], r2[w], 0x05040100u));
      const uint2 odd = make_uint2(perm(r1[w], r0[w], 0x07060302u), perm(r3[w], r2[w], 0x07060302u));
      const int d = 8 * oc + 2 * w;
      *reinterpret_cast<uint2*>(&s.vt[d * Smem<D>::vStride + 4 * kq]) = even;
      *reinterpret_cast<uint2*>(&s.vt[(d + 1) * Smem<D>::vStride + 4 * kq]) = odd;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p, int n_mtiles) {
  constexpr int KS = D / 16;  // k-steps of 16 over the head dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  __shared__ Smem<D> sbuf[2];  // double buffer: tile i computes from one while i+1 is stored

  // XCD-aware work mapping (see header).
  const int total = (int)(gridDim.x);
  const int bid = blockIdx.x;
  const int work = (total % kXcds == 0) ? (bid % kXcds) * (total / kXcds) + bid / kXcds : bid;
  const int mt_rev = work % n_mtiles;
  const int h = (work / n_mtiles) % p.num_q_heads;
  const int prompt = work / (n_mtiles * p.num_q_heads);
  const int mt = n_mtiles - 1 - mt_rev;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = h / G;

  const int q0 = p.cu_seqlens_q[prompt];
  const int q1 = p.cu_seqlens_q[prompt + 1];
  if (q0 < 0 || q1 < q0 || q1 > p.q_rows) return;  // rows not addressable: nothing to write
  const int L = q1 - q0;
  const int m0 = mt * kM;
  const int kv0 = p.kv_start[prompt];
  const bool ok = L <= p.max_len && kv0 >= 0 && (int64_t)kv0 + L <= p.kv_rows;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int r0 = m0 + 32 * wave;     // first row (position in prompt) of this wavefront
  const int qpos = r0 + col;         // the query this lane's column holds
  const int64_t qrow = (int64_t)q0 + qpos;
  const int64_t hq_row = (int64_t)p.num_q_heads * D;

  if (!ok) {  // offsets outside the buffers or an over-long prompt: row tile 0 writes NaN rows
    if (mt != 0) return;
    const float qnan = __builtin_nanf("");
    for (int64_t i = threadIdx.x; i < (int64_t)L * D; i += kThreads) {
      const int64_t rr = i / D;
      const int64_t o = ((int64_t)q0 + rr) * hq_row + (int64_t)h * D + i % D;
      if (p.out_f32) static_cast<float*>(p.out)[o] = qnan;
      else static_cast<f16*>(p.out)[o] = (f16)qnan;
      if (p.lse && i % D == 0) p.lse[((int64_t)q0 + rr) * p.num_q_heads + h] = qnan;
    }
    return;
  }

  if (m0 >= L) return;

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

  const int n_end = p.causal ? min(L, m0 + kM) : L;
  const int n_tiles = (n_end + kN - 1) / kN;
  // buffer descriptors over this prompt's K/V rows of KV head g
  const uint32_t rowb = (uint32_t)p.num_kv_heads * D * 2u;  // bytes per key row
  const uint32_t span = (uint32_t)(L - 1) * rowb + D * 2u;
  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)kv0 * p.num_kv_heads + g) * D * 2;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)kv0 * p.num_kv_heads + g) * D * 2;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, span, kBufferFlags);
  uint32_t koff[TileRegs<D>::KCH], voff[4];
#pragma unroll
  for (int i = 0; i < TileRegs<D>::KCH; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    koff[i] = (uint32_t)(idx / (D / 8)) * rowb + 16u * (idx % (D / 8));
  }
  {
    constexpr int units = (kN / 4) * (D / 8);
    const int t = threadIdx.x < units ? threadIdx.x : 0;
    const int kq = t % (kN / 4), oc = t / (kN / 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)(4 * kq + i) * rowb + 16u * oc;
  }
  TileRegs<D> tr;
  load_tile<D>(tr, kr, vr, koff, voff, 0u);
  store_tile<D>(sbuf[0], tr);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int n0 = it * kN;
    Smem<D>& s = sbuf[it & 1];
    // the next tile's loads are in flight while this tile computes
    if (it + 1 < n_tiles) load_tile<D>(tr, kr, vr, koff, voff, (uint32_t)(n0 + kN) * rowb);

    if (!(p.causal && n0 > r0 + 31)) {  // skip tiles whose keys all follow this wavefront's rows

    // S^T = K . Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const f16* kp = &s.k[(kb * 32 + col) * Smem<D>::kStride + 8 * half];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(kp + 16 * ks);
        sacc[kb] = mfma32(a, qb[ks], sacc[kb]);
      }
    }

    // mask (causal diagonal, prompt end) on the raw scores; the log2-unit scale
    // is folded into the exponent's fma below (scale > 0 keeps the max)
    const bool need_mask = (p.causal && n0 + kN - 1 > r0) || (n0 + kN > L);
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kb][r];
        if (need_mask) {
          const int key = n0 + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          const bool vis = key < L && (!p.causal || key <= qpos);
          x = vis ? x : -__builtin_inff();
        }
        sacc[kb][r] = x;
        mx = fmaxf(mx, x);
      }
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

    // P^T operand (fp16): PV k-block kk uses registers 8(kk%2)..+8 of block kk/2
    f16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(__builtin_fmaf(sacc[kb][r], p.scale_log2, -m));
        l += pv;
        pb[kb * 2 + r / 8][r % 8] = (f16)pv;
      }
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f16* vp = &s.vt[(32 * db + col) * Smem<D>::vStride + 4 * half];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vp + 16 * kk);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16 * kk + 8);
        const uint4 a4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[db] = mfma32(__builtin_bit_cast(f16x8, a4), pb[kk], oacc[db]);
      }
    }
    }
    // store the next tile into the other buffer; one barrier publishes it and
    // guarantees every wavefront has finished reading the buffer it overwrites next
    if (it + 1 < n_tiles) store_tile<D>(sbuf[(it + 1) & 1], tr);
    __syncthreads();
  }

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

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.n_prompts == 0 || p.max_len == 0) return hipSuccess;
  const int n_mtiles = (p.max_len + kM - 1) / kM;
  const int64_t blocks = (int64_t)n_mtiles * p.num_q_heads * p.n_prompts;
  if (p.head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, n_mtiles);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, n_mtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ekv

// Compact-page gather: K16/V8 pages -> contiguous FP16 workspace.
//
// Source: "Memory-Traffic Saturation in Autoregressive Transformer Decode",
// section "What changes in vLLM's prefill routing?" (figure "Fresh prefill
// gets a fast path inside a mixed batch"): stored K16/V8 pages are gathered
// into one bounded FP16 workspace and V8 is cast to FP16 for the prefill.
//
// HBM-bound: per element 3 B read (K16 + V8) and 4 B written.  One thread
// moves one 16-element run of one page (16 V bytes, 32 K bytes in, 64 B
// out) with 16-byte vector accesses; consecutive threads cover consecutive
// runs of a page, so every access of a wavefront is a contiguous 1 KiB span.
#include "ekv_device.hpp"
#include "ekv_internal.hpp"

namespace ekv {
namespace {

constexpr int kGatherThreads = 256;

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 under the default mode).
__device__ __forceinline__ uint32_t pack_rne(float a, float b) {
  f16x2 r;
  r.x = (f16)a;
  r.y = (f16)b;
  return bits(r);
}

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherParams p) {
#pragma clang fp contract(off)
  const int runs_per_page = p.num_kv_heads * p.head_dim;  // 16 slots * Hkv * D / 16
  const int64_t run = (int64_t)blockIdx.x * kGatherThreads + threadIdx.x;
  if (run >= (int64_t)p.n_pages * runs_per_page) return;
  const int page = (int)(run / runs_per_page);
  const int w = (int)(run - (int64_t)page * runs_per_page);
  const int64_t elem = (int64_t)w * 16;                     // element offset inside the page
  const int head = (int)((elem / p.head_dim) % p.num_kv_heads);
  const int64_t page_elems = (int64_t)kPage * p.num_kv_heads * p.head_dim;
  const int64_t dst = (int64_t)page * page_elems + elem;
  uint4* dk = reinterpret_cast<uint4*>(p.ws_k + dst);
  uint4* dv = reinterpret_cast<uint4*>(p.ws_v + dst);

  const int id = p.page_ids[page];
  if ((unsigned)id >= (unsigned)p.n_pool) {
    const uint32_t nan2 = (uint32_t)kF16NaN | ((uint32_t)kF16NaN << 16);
    const uint4 nan4 = make_uint4(nan2, nan2, nan2, nan2);
    dk[0] = nan4; dk[1] = nan4; dv[0] = nan4; dv[1] = nan4;
    return;
  }
  const int64_t src = (int64_t)id * page_elems + elem;
  const uint4* sk = reinterpret_cast<const uint4*>(p.k_compact + src);
  const uint4 k0 = sk[0];
  const uint4 k1 = sk[1];
  const uint4 v8 = *reinterpret_cast<const uint4*>(p.v_compact + src);
  const float s = p.apply_scale ? p.v_scale[(int64_t)id * p.num_kv_heads + head] : 1.0f;

  const uint32_t in[4] = {v8.x, v8.y, v8.z, v8.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 a = e4m3x2_f32(in[i], false);  // exact
    const f32x2 b = e4m3x2_f32(in[i], true);
    o[2 * i] = pack_rne(a.x * s, a.y * s);     // one fp32 RNE multiply, one fp16 RNE
    o[2 * i + 1] = pack_rne(b.x * s, b.y * s);
  }
  dk[0] = k0;
  dk[1] = k1;
  dv[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dv[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// Diagnostic: code * 2^scale_exp to fp16.  method 0 = the conversion the
// decode kernel uses (4 codes per word, both word halves, the instruction's
// power-of-two scale); method 1 = the gather's arithmetic (exact fp32 value
// times the fp32 scale, rounded to nearest even, then to fp16 nearest even).
__global__ void e4m3_to_f16_kernel(const uint8_t* codes, int32_t n, uint16_t* out, int32_t method,
                                   int32_t scale_exp) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i >= n) return;
  uint32_t w = 0;
  for (int k = 0; k < 4 && 4 * i + k < n; ++k) w |= (uint32_t)codes[4 * i + k] << (8 * k);
  const float s = __builtin_amdgcn_ldexpf(1.0f, scale_exp);
  uint32_t r[2];
  if (method == 1) {
#pragma clang fp contract(off)
    const f32x2 a = e4m3x2_f32(w, false), b = e4m3x2_f32(w, true);
    r[0] = pack_rne(a.x * s, a.y * s);
    r[1] = pack_rne(b.x * s, b.y * s);
  } else {
    r[0] = bits(e4m3x2_scaled_f16(w, s, false));
    r[1] = bits(e4m3x2_scaled_f16(w, s, true));
  }
  for (int k = 0; k < 4 && 4 * i + k < n; ++k) out[4 * i + k] = (uint16_t)(r[k / 2] >> (16 * (k % 2)));
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  const int64_t runs = (int64_t)p.n_pages * p.num_kv_heads * p.head_dim;
  if (runs == 0) return hipSuccess;
  const int64_t blocks = (runs + kGatherThreads - 1) / kGatherThreads;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(kGatherThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_e4m3_to_f16(const uint8_t* codes, int32_t n, uint16_t* out, int32_t method,
                              int32_t scale_exp, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(e4m3_to_f16_kernel, dim3((n + 1023) / 1024), dim3(256), 0, stream, codes, n,
                     out, method, scale_exp);
  return hipGetLastError();
}

}  // namespace ekv

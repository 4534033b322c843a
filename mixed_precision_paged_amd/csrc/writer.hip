// Cache writer: token append into TARGET pages, and compact-page quantization.
//
// Sources: "Does Execution Require Target KV Fidelity? ..." (ElasticKV)
// section 3.2 and appendix B.3 (new KV is stored at target fidelity in the
// protected recent window) and section 3.3 (a demotion rewrites whole pages);
// "Memory-Traffic Saturation in Autoregressive Transformer Decode", section
// "What changes in vLLM's prefill routing?" and the table "Historical reported
// implementation checks" (the cache writer keeps K bit for bit and holds V
// as E4M3 codes with value scales).
//
// Both kernels are HBM-bound copies with a little ALU work:
//   append:   per token, 4 B read and 4 B written per (K, V) element pair;
//   quantize: per page, 4 B read (K16 + V16) and 3 B written (K16 + E4M3 V)
//             per pair, plus one fp32 scale per (page, KV head).
// One wavefront owns one unit (a token row, or one KV head of one page), so
// every per-unit index is wave-uniform and lives in scalar registers.
#include "ekv_device.hpp"
#include "ekv_internal.hpp"

namespace ekv {
namespace {

constexpr int kWriterThreads = 256;
constexpr int kWriterWaves = kWriterThreads / kWave;
// Buffer cache policy of the quantizer's row loads and page stores: each
// byte is moved once (non-temporal, evict first; loads and stores together
// measured 2% faster than the default, either alone no faster).
constexpr int kNonTemporalAux = 2;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Append: token t's K and V rows (all KV heads) -> TARGET slot slot_mapping[t]
// (slot = page * 16 + index in page).  Negative or out-of-pool slots are
// skipped.
__global__ __launch_bounds__(kWriterThreads) void append_kernel(AppendParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kWriterWaves + wave;
  if (t >= p.n_tokens) return;
  const int slot = __builtin_amdgcn_readfirstlane(p.slot_mapping[t]);
  if (slot < 0 || (int64_t)slot >= (int64_t)p.n_target * kPage) return;
  const int chunks = p.num_kv_heads * p.head_dim / 8;  // 16-byte chunks per row
  const int64_t src = t * (int64_t)p.num_kv_heads * p.head_dim;
  const int64_t dst = (int64_t)slot * p.num_kv_heads * p.head_dim;
  const uint4* sk = reinterpret_cast<const uint4*>(p.k_new + src);
  const uint4* sv = reinterpret_cast<const uint4*>(p.v_new + src);
  uint4* dk = reinterpret_cast<uint4*>(p.k_target + dst);
  uint4* dv = reinterpret_cast<uint4*>(p.v_target + dst);
  for (int c = lane; c < chunks; c += kWave) {
    // new rows are read once: non-temporal loads (26% faster than the default)
    const u32x4 kn = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sk) + c);
    const u32x4 vn = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sv) + c);
    const uint4 k = make_uint4(kn.x, kn.y, kn.z, kn.w), v = make_uint4(vn.x, vn.y, vn.z, vn.w);
    dk[c] = k;
    dv[c] = v;
  }
}

// ---------------------------------------------------------------------------
// fp32 -> E4M3FN code, nearest value with ties to the even mantissa,
// saturating at 448, NaN -> 0x7F.  Normal range (|x| >= 2^-6): re-bias the
// fp32 exponent from 127 to 7 and round the 23-bit mantissa to 3 bits in
// integer arithmetic (a carry moves into the exponent as it should).
// Subnormal range: the value grid is k * 2^-9, k = 0..8, so round x * 2^9 to
// an integer (exact scaling, v_rndne_f32 ties to even); k = 8 is code 0x08.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t r = a - (120u << 23);
  uint32_t normal = (r + 0x7FFFFu + ((r >> 20) & 1u)) >> 20;
  normal = normal < 0x7Eu ? normal : 0x7Eu;
  const uint32_t sub = (uint32_t)__builtin_rintf(as_f32(a) * 512.0f);
  const uint32_t code = (a >= 0x3C800000u ? normal : sub) | sign;
  return a > 0x7F800000u ? 0x7Fu : code;
}

// Correctly rounded fp32 quotient v / s from y = RN(1/s): two FMA correction
// steps (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Dev. 34(1), 1990): the first makes the
// quotient faithful, the second rounds it correctly.  No overflow or
// underflow is possible here: |v / s| <= 448 (1 + 2^-23) and |v| >= 2^-24.
// With s > 0 the quotient has the sign of v; restoring it keeps -0 / s = -0
// (the correction sums of opposite zeros round to +0).
__device__ __forceinline__ float div_rn(float v, float s, float y) {
  float q = v * y;
  q = __builtin_fmaf(__builtin_fmaf(-s, q, v), y, q);
  q = __builtin_fmaf(__builtin_fmaf(-s, q, v), y, q);
  return __builtin_copysignf(q, v);
}

__device__ __forceinline__ uint32_t absmax_u16x2(uint32_t m, uint32_t x) {
  const u16x2 a = __builtin_bit_cast(u16x2, x & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m), a));
}

// Four fp16 values (two words) -> four codes packed in one word, byte k = element k.
__device__ __forceinline__ uint32_t encode4(uint32_t w0, uint32_t w1, float s, float y) {
  const f16x2 a = as_f16x2(w0), b = as_f16x2(w1);
  const uint32_t c0 = e4m3_encode(div_rn((float)a.x, s, y));
  const uint32_t c1 = e4m3_encode(div_rn((float)a.y, s, y));
  const uint32_t c2 = e4m3_encode(div_rn((float)b.x, s, y));
  const uint32_t c3 = e4m3_encode(div_rn((float)b.y, s, y));
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// One wave per (page i, KV head h).  Lane l covers 16-byte chunk l % (D/8)
// of rows l / (D/8) + (64 / (D/8)) * j.  Source rows past n_valid lie past
// the end of the source descriptor's range and read as zero, which is the
// content the page gets there (K +0.0, code 0x00).
template <int D>
__global__ __launch_bounds__(kWriterThreads) void quantize_kernel(QuantizeParams p) {
  constexpr int kCpr = D / 8;            // chunks per row
  constexpr int kRpp = kWave / kCpr;     // rows per pass
  constexpr int kPasses = kPage / kRpp;  // 4 (D = 128) or 2 (D = 64)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t unit = (int64_t)blockIdx.x * kWriterWaves + wave;
  if (unit >= (int64_t)p.n_pages * p.num_kv_heads) return;
  const int i = (int)(unit / p.num_kv_heads);
  const int h = (int)(unit - (int64_t)i * p.num_kv_heads);
  const int row0 = __builtin_amdgcn_readfirstlane(p.src_row_start[i]);
  const int n = p.n_valid ? __builtin_amdgcn_readfirstlane(p.n_valid[i]) : kPage;
  const int dst = __builtin_amdgcn_readfirstlane(p.dst_pages[i]);
  if (row0 < 0 || n < 0 || n > kPage || (int64_t)row0 + n > p.src_rows) return;
  if (dst < 0 || dst >= p.n_compact) return;

  const int row_elems = p.num_kv_heads * D;
  const uint32_t row_bytes = (uint32_t)row_elems * 2u;
  const int64_t src_off = (int64_t)row0 * row_elems + (int64_t)h * D;
  const uint32_t src_bytes = (uint32_t)n * row_bytes;
  const __amdgpu_buffer_rsrc_t ks =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_src + src_off), (short)0, src_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v_src + src_off), (short)0, src_bytes, kBufferFlags);
  const int64_t dst_off = (int64_t)dst * kPage * row_elems + (int64_t)h * D;
  const uint32_t kd_bytes = 15u * row_bytes + D * 2u;
  const uint32_t vd_bytes = 15u * (uint32_t)row_elems + D;
  const __amdgpu_buffer_rsrc_t kd =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_compact + dst_off), (short)0, kd_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vd =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v_compact + dst_off), (short)0, vd_bytes, kBufferFlags);

  const int c = lane % kCpr;
  const int r0 = lane / kCpr;
  const uint32_t off16 = (uint32_t)r0 * row_bytes + 16u * c;          // fp16 rows
  const uint32_t off8 = (uint32_t)r0 * (uint32_t)row_elems + 8u * c;  // code rows

  u32x4 v[kPasses];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    const u32x4 k = __builtin_amdgcn_raw_buffer_load_b128(ks, off16, j * kRpp * row_bytes, kNonTemporalAux);
    v[j] = __builtin_amdgcn_raw_buffer_load_b128(vs, off16, j * kRpp * row_bytes, kNonTemporalAux);
    __builtin_amdgcn_raw_buffer_store_b128(k, kd, off16, j * kRpp * row_bytes, kNonTemporalAux);
  }
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    m = absmax_u16x2(m, v[j].x);
    m = absmax_u16x2(m, v[j].y);
    m = absmax_u16x2(m, v[j].z);
    m = absmax_u16x2(m, v[j].w);
  }
  m = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
#pragma unroll
  for (int x = 1; x < kWave; x <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, x, kWave);
    m = o > m ? o : m;
  }
  const float absmax = (float)__builtin_bit_cast(f16, (uint16_t)m);
  const float s = m ? absmax / 448.0f : 1.0f;  // correctly rounded fp32 division
  const float y = 1.0f / s;                    // RN(1/s)
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    u32x2 w;
    w.x = encode4(v[j].x, v[j].y, s, y);
    w.y = encode4(v[j].z, v[j].w, s, y);
    __builtin_amdgcn_raw_buffer_store_b64(w, vd, off8, j * kRpp * (uint32_t)row_elems, kNonTemporalAux);
  }
  if (lane == 0) p.v_scale[(int64_t)dst * p.num_kv_heads + h] = s;
}

// ---------------------------------------------------------------------------
// ElasticKV demotion pack: pair i's TARGET blocks src_a[i], src_b[i] -> block
// dst[i] holding their high bytes (half 0 = a, half 1 = b), i.e. BASE pages
// 2 dst and 2 dst + 1.  One workgroup per (pair, pool): every thread reads its
// 16-byte chunks of both blocks and keeps their high bytes; a barrier; then
// the writes, so dst may be a or b (in place).  blockIdx.y: 0 = K pool, 1 = V.
constexpr int kPackMaxUnits = 8;  // 32-byte units of one block per thread (Hkv*D <= 2048)

__global__ __launch_bounds__(kWriterThreads) void pack_base_kernel(PackParams p) {
  const int pair = blockIdx.x;
  char* pool = reinterpret_cast<char*>(blockIdx.y == 0 ? p.k_target : p.v_target);
  const int a = p.src_a[pair], b = p.src_b[pair], d = p.dst[pair];
  if ((unsigned)a >= (unsigned)p.n_target || (unsigned)b >= (unsigned)p.n_target ||
      (unsigned)d >= (unsigned)p.n_target)
    return;  // uniform for the workgroup: nothing is read or written
  // a unit = 16 fp16 values (32 bytes) of a source block -> their 16 high
  // bytes, one 16-byte store into each half of the destination block
  const int units = kPage * p.num_kv_heads * p.head_dim / 16;
  const int64_t block_bytes = (int64_t)units * 32;
  const uint4* pa = reinterpret_cast<const uint4*>(pool + a * block_bytes);
  const uint4* pb = reinterpret_cast<const uint4*>(pool + b * block_bytes);
  uint4 ha[kPackMaxUnits], hb[kPackMaxUnits];
#pragma unroll
  for (int j = 0; j < kPackMaxUnits; ++j) {
    const int c = threadIdx.x + kWriterThreads * j;
    if (c < units) {
      // each source block is read once: non-temporal loads (20% faster)
      const u32x4 x0n = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pa) + 2 * c);
      const u32x4 x1n = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pa) + 2 * c + 1);
      const u32x4 y0n = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pb) + 2 * c);
      const u32x4 y1n = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pb) + 2 * c + 1);
      const uint4 x0 = make_uint4(x0n.x, x0n.y, x0n.z, x0n.w), x1 = make_uint4(x1n.x, x1n.y, x1n.z, x1n.w);
      const uint4 y0 = make_uint4(y0n.x, y0n.y, y0n.z, y0n.w), y1 = make_uint4(y1n.x, y1n.y, y1n.z, y1n.w);
      // bytes 1, 3, 5, 7 of each 8-byte half: the high bytes of 4 fp16 values
      ha[j] = make_uint4(perm(x0.y, x0.x, 0x07050301u), perm(x0.w, x0.z, 0x07050301u),
                         perm(x1.y, x1.x, 0x07050301u), perm(x1.w, x1.z, 0x07050301u));
      hb[j] = make_uint4(perm(y0.y, y0.x, 0x07050301u), perm(y0.w, y0.z, 0x07050301u),
                         perm(y1.y, y1.x, 0x07050301u), perm(y1.w, y1.z, 0x07050301u));
    }
  }
  __syncthreads();
  uint4* out0 = reinterpret_cast<uint4*>(pool + d * block_bytes);
  uint4* out1 = reinterpret_cast<uint4*>(pool + d * block_bytes + block_bytes / 2);
#pragma unroll
  for (int j = 0; j < kPackMaxUnits; ++j) {
    const int c = threadIdx.x + kWriterThreads * j;
    if (c < units) {
      out0[c] = ha[j];
      out1[c] = hb[j];
    }
  }
}

}  // namespace

hipError_t launch_pack_base(const PackParams& p, hipStream_t stream) {
  if (p.n_pairs == 0) return hipSuccess;
  if (kPage * p.num_kv_heads * p.head_dim / 16 > kPackMaxUnits * kWriterThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_base_kernel, dim3((unsigned)p.n_pairs, 2), dim3(kWriterThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  if (p.n_tokens == 0) return hipSuccess;
  const int64_t blocks = (p.n_tokens + kWriterWaves - 1) / kWriterWaves;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kWriterThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.n_pages * p.num_kv_heads;
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + kWriterWaves - 1) / kWriterWaves;
  if (p.head_dim == 128)
    hipLaunchKernelGGL(quantize_kernel<128>, dim3((unsigned)blocks), dim3(kWriterThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(quantize_kernel<64>, dim3((unsigned)blocks), dim3(kWriterThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ekv

// Device helpers shared by the HIP kernels of libekv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ekv {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a gfx9 raw buffer descriptor (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

constexpr int kPage = 16;
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint16_t kF16NaN = 0x7E00;

__device__ __forceinline__ uint32_t bits(f16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// Byte permute of the 8-byte value {hi:lo}: selector byte k picks byte k of
// (lo = bytes 0..3, hi = bytes 4..7) for result byte k.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// DPP lane moves inside a wavefront (gfx9 encodings).
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <- lane 7-i inside each 8-lane half row
  kDppRowRor8 = 0x128,    // lane i <- lane (i+8) mod 16 inside each 16-lane row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 8 lanes of an aligned lane octet; every lane gets the sum.
__device__ __forceinline__ float octet_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

// Two E4M3FN codes (word half `hi`) -> two fp16 values of code * scale,
// via the gfx950 scaled conversion.  With scale 1.0 the result is exact.
__device__ __forceinline__ f16x2 e4m3x2_scaled_f16(uint32_t w, float scale, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, scale, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, scale, false);
}

// Two E4M3FN codes (word half `hi`) -> two exact fp32 values.
__device__ __forceinline__ f32x2 e4m3x2_f32(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_f16x2(a), as_f16x2(b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace ekv

// Internal device helpers shared by the libcsa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int D = CSA_D;                 // latent width
constexpr int HEADS = CSA_HEADS;         // attention query heads
constexpr int IH = CSA_IDX_HEADS;        // indexer heads
constexpr int ID = CSA_IDX_DIM;          // indexer head width
constexpr int CODE_BYTES = CSA_CODE_BYTES;
constexpr int SCALE_BYTES = CSA_SCALE_BYTES;
constexpr int NWIN = CSA_N_WIN;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ E4M3FN ------
// Value of the non-negative E4M3FN code c in 0..126 (exact in fp32):
// exponent field e (bias 7), mantissa m; e = 0 is subnormal m/8 * 2^-6.
__device__ __forceinline__ float e4m3_code_value(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// RNE_E4M3FN(a / f) for a >= 0 and f in {1, 6}, saturating at 448.
// Exact: it counts the rounding midpoints mid_i (between codes i and i+1)
// with f * mid_i < a; f * mid_i has at most 7 significant bits, so it and the
// comparisons are exact in fp32.  A tie (a == f * mid_i) goes to the even code.
__device__ __forceinline__ uint32_t e4m3_rne_div(float a, float f) {
  uint32_t lo = 0;
#pragma unroll
  for (uint32_t step = 64; step >= 1; step >>= 1) {
    uint32_t c = lo + step;              // test midpoint c-1 (between c-1 and c)
    if (c <= 126u) {
      float mid = 0.5f * (e4m3_code_value(c - 1) + e4m3_code_value(c));
      if (f * mid < a) lo = c;
    }
  }
  if (lo < 126u && (lo & 1u)) {
    float mid = 0.5f * (e4m3_code_value(lo) + e4m3_code_value(lo + 1));
    if (f * mid == a) lo += 1;
  }
  return lo;
}

// Signed E4M3FN encode of x (RNE, saturating, sign bit of x kept).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t mag = e4m3_rne_div(fabsf(x), 1.0f);
  return mag | ((__float_as_uint(x) >> 24) & 0x80u);
}

// ------------------------------------------------------------ MXFP4 -------
// One 16-channel group: scale byte s = RNE_E4M3(amax / 6), codes
// signbit << 3 | RNE_E2M1(|x| / s) (saturating at 6, ties to the even code).
// The element decision compares |x| with s * midpoint (exact products), so
// no division is performed.  Returns the scale byte; codes8 receives the 16
// nibbles packed channel-2k-low into 8 bytes (two dwords).
__device__ __forceinline__ uint32_t mxfp4_group(const float* v, uint32_t codes8[2]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t sc = e4m3_rne_div(amax, 6.0f);
  float s = e4m3_code_value(sc);
  float t0 = s * 0.25f, t1 = s * 0.75f, t2 = s * 1.25f, t3 = s * 1.75f;
  float t4 = s * 2.5f, t5 = s * 3.5f, t6 = s * 5.0f;
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float r = fabsf(v[i]);
    // threshold k lies between codes k and k+1; a tie rounds to the even one
    uint32_t c = (uint32_t)(r > t0) + (uint32_t)(r >= t1) + (uint32_t)(r > t2) +
                 (uint32_t)(r >= t3) + (uint32_t)(r > t4) + (uint32_t)(r >= t5) +
                 (uint32_t)(r > t6);
    c = (sc == 0u) ? 0u : c;
    c |= (__float_as_uint(v[i]) >> 28) & 0x8u;
    if (i < 8) w0 |= c << (4 * i);
    else w1 |= c << (4 * (i - 8));
  }
  codes8[0] = w0;
  codes8[1] = w1;
  return sc;
}

// E2M1 magnitude of a 3-bit code (exact): 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  c &= 7u;
  if (c < 2u) return 0.5f * (float)c;
  return __uint_as_float(((c >> 1) + 126u) << 23 | ((c & 1u) << 22));
}

// ------------------------------------------------------- fp16 unpacking ----
// Two E2M1 codes (low / high nibble of byte `sel` of w) -> fp16 pair, exact.
// The gfx950 conversion is used with scale 1.0 (exact for every code).
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// Two E4M3FN bytes (word `SEL` of w) -> fp16 pair, exact.
template <int SEL>
__device__ __forceinline__ f16x2 fp8x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t f16x2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 bits_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// Key of a float for descending selection: larger key = larger value.
// -inf and NaN map to 0 (never selected); -0 maps like +0.
__device__ __forceinline__ uint32_t select_key(float x) {
  if (!(x > -__builtin_huge_valf())) return 0u;
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// MFMA wrappers (layouts verified: C lane l holds rows 4*(l/16)+r, column l%16).
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// fp64 16x16x4: A lane l = row l%16, k l/16 (same as fp32), but the result
// lane l, register r holds row l/16 + 4r, column l%16 (verified on gfx950).
__device__ __forceinline__ f64x4 mfma_f64_16x16x4(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int visible_count(int32_t pos) { return pos < 0 ? 0 : (pos + 1) >> 2; }

}  // namespace csa

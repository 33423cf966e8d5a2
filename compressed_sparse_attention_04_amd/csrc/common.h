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

// Non-negative E4M3FN code of RNE(v), saturating at 448 (v >= 0; NaN -> 0).
// Normal range: v = f * 2^E, f in [1, 2): mantissa = rint((f - 1) * 8), a
// carry to 8 moves to the next exponent; below 2^-6 the code is rint(v * 2^9)
// (8 there is the smallest normal, code 0x08).  rint rounds half to even, and
// the even integer is the code whose last bit is 0.  All steps are exact.
__device__ __forceinline__ uint32_t e4m3_rne_f64(double v) {
  if (!(v > 0.0)) return 0u;
  if (v >= 448.0) return 0x7Eu;
  if (v < 0x1p-6) return (uint32_t)rint(v * 512.0);
  int e;
  double f = frexp(v, &e);                 // v = f * 2^e, f in [0.5, 1)
  int E = e - 1;
  uint32_t m = (uint32_t)rint((2.0 * f - 1.0) * 8.0);
  if (m == 8u) { m = 0u; E += 1; }
  uint32_t c = ((uint32_t)(E + 7) << 3) | m;
  return c > 0x7Eu ? 0x7Eu : c;
}
__device__ __forceinline__ uint32_t e4m3_rne_f32(float v) {
  if (!(v > 0.f)) return 0u;
  if (v >= 448.f) return 0x7Eu;
  if (v < 0x1p-6f) return (uint32_t)rintf(v * 512.f);
  int e;
  float f = frexpf(v, &e);
  int E = e - 1;
  uint32_t m = (uint32_t)rintf((2.f * f - 1.f) * 8.f);
  if (m == 8u) { m = 0u; E += 1; }
  uint32_t c = ((uint32_t)(E + 7) << 3) | m;
  return c > 0x7Eu ? 0x7Eu : c;
}

// Scale code RNE_E4M3(amax / 6): the quotient is formed in fp64, which takes
// the same rounding decision as exact division (amax has 24 significant bits,
// 6 and every E4M3 midpoint at most 5, so a quotient that is not exactly a
// midpoint is at least ~2^-24 relative away from one; fp64 errs by 2^-53).
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax) {
  return e4m3_rne_f64((double)amax / 6.0);
}

// Signed E4M3FN encode of x (RNE, saturating, sign bit of x kept).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t mag = e4m3_rne_f32(fabsf(x));
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
  uint32_t sc = e4m3_scale_code(amax);
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

// One element's 4-bit code under scale value s (scale code sc): sign bit of x,
// magnitude RNE_E2M1(|x| / s) decided by comparing |x| with s * midpoints.
__device__ __forceinline__ uint32_t e2m1_code(float x, float s, uint32_t sc) {
  float r = fabsf(x);
  uint32_t c = (uint32_t)(r > s * 0.25f) + (uint32_t)(r >= s * 0.75f) + (uint32_t)(r > s * 1.25f) +
               (uint32_t)(r >= s * 1.75f) + (uint32_t)(r > s * 2.5f) + (uint32_t)(r >= s * 3.5f) +
               (uint32_t)(r > s * 5.0f);
  c = (sc == 0u) ? 0u : c;
  return c | ((__float_as_uint(x) >> 28) & 0x8u);
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

// ------------------------------------------------------ cross-lane steps ----
// VALU-only exchanges (no LDS round trip).  gfx950's v_permlane16_swap with
// both operands = v returns {rows 0,0,2,2 ; rows 1,1,3,3} of v (16-lane rows),
// v_permlane32_swap {lanes 0-31 twice ; lanes 32-63 twice}; combining the two
// halves is an xor-16 / xor-32 reduction with the lower row's value first.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max(a, b) for non-NaN floats as gfx950's v_maximum3_f32 (IEEE maximum,
// NaN-propagating): fmaxf would first quiet both inputs (two more
// instructions).
__device__ __forceinline__ float fmax_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max over each aligned group of 8 lanes, in every lane of the group (DPP:
// quad_perm xor 1, xor 2, then row_half_mirror, which pairs the two quads).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  return fmaxf(v, dpp_f<0x141>(v));
}

// Key of a float for descending selection: larger key = larger value.
// -inf and NaN map to 0 (never selected); -0 maps like +0.
__device__ __forceinline__ uint32_t select_key(float x) {
  if (!(x > -__builtin_huge_valf())) return 0u;
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// MFMA wrappers (layouts verified: C lane l holds rows 4*(l/16)+r, column l%16).
__device__ __forceinline__ f32x4 mfma_f16_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// fp64 16x16x4: A lane l = row l%16, k l/16 (same as fp32), but the result
// lane l, register r holds row l/16 + 4r, column l%16 (verified on gfx950).
__device__ __forceinline__ f64x4 mfma_f64_16x16x4(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int visible_count(int32_t pos) { return pos < 0 ? 0 : (pos + 1) >> 2; }

}  // namespace csa

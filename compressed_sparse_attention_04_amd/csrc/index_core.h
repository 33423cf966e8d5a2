// Indexer fragment routines (E4M3 operands widened to fp16, 16 x 16 x 32
// MFMA fragments, weighted ReLU head sum), shared by the scoring kernels and
// the fused Full-layer kernel.  The method is described in index.hip.
#pragma once

#include "common.h"

namespace csa {
namespace idxf {

// One lane's share of a 16 x 128 operand fragment: 32 E4M3 bytes of one row,
// bytes 16 g .. 16 g + 15 (u0) and 64 + 16 g .. 64 + 16 g + 15 (u1) with
// g = lane / 16.  A and B use the same byte -> k mapping (k-steps 0, 1 take
// u0, k-steps 2, 3 take u1), so the four 16x16x32 products contract exactly
// the 128 channels.
struct Raw32 { uint4 u0, u1; };
struct Frag16 { f16x8 s[4]; };

__device__ __forceinline__ Raw32 load_raw32(const uint8_t* row, bool live, int lane) {
  Raw32 r = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
  if (live) {
    const uint4* p = reinterpret_cast<const uint4*>(row + 16 * (lane >> 4));
    r.u0 = p[0];
    r.u1 = p[4];
  }
  return r;
}

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  if (NT) {
    const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
  }
  return *reinterpret_cast<const uint4*>(p);
}

// Key fragments are loaded whole-line and transposed through LDS: half h of a
// 16-row fragment (rows 8h .. 8h+7, 1 KB) is one load instruction in which
// lane i reads 16-byte chunk (i % 8) ^ (n / 2) of row n = 8h + i / 8 and
// stores it to staging slot 64h + i.  Row n's chunk c therefore sits in slot
// 8n + (c ^ (n / 2)): the stores are contiguous and the 16 rows a read
// instruction touches fall in 16 distinct bank groups.
__device__ __forceinline__ int stage_chunk(int lane, int h) { return (lane & 7) ^ ((8 * h + (lane >> 3)) >> 1); }
__device__ __forceinline__ Raw32 read_staged(const uint4* stage, int lane) {
  const int n = lane & 15, g = lane >> 4, sw = n >> 1;
  Raw32 r;
  r.u0 = stage[8 * n + (g ^ sw)];
  r.u1 = stage[8 * n + ((4 + g) ^ sw)];
  return r;
}

__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t w0, uint32_t w1) {
  f16x2 a = fp8x2_to_f16<0>(w0), b = fp8x2_to_f16<1>(w0);
  f16x2 c = fp8x2_to_f16<0>(w1), d = fp8x2_to_f16<1>(w1);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ Frag16 to_frag(const Raw32& r) {
  Frag16 f;
  f.s[0] = fp8x8_to_f16(r.u0.x, r.u0.y);
  f.s[1] = fp8x8_to_f16(r.u0.z, r.u0.w);
  f.s[2] = fp8x8_to_f16(r.u1.x, r.u1.y);
  f.s[3] = fp8x8_to_f16(r.u1.z, r.u1.w);
  return f;
}

__device__ __forceinline__ f32x4 frag_mma(const Frag16& a, const Frag16& b) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f16_16x16x32(a.s[s], b.s[s], acc);
  return acc;
}

// A fragment of (query q, head) for this lane; zero when the row is absent.
__device__ __forceinline__ Frag16 load_qfrag(const uint8_t* q_fp8, int64_t q, int head, bool live,
                                             int lane) {
  return to_frag(load_raw32(q_fp8 + (q * IH + head) * ID, live, lane));
}

// ReLU on the bit pattern: a float with the sign bit set is a negative int32,
// so max(bits, 0) maps every negative (and -0) to +0 and keeps the rest; one
// integer max, where fmaxf would also have to quiet its inputs.
__device__ __forceinline__ float relu(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// Weighted ReLU head sum of one accumulator fragment.  head_part is the
// lane's sum over its 4 rows; head_sum adds the other half of the 8 heads, so
// lanes 0-15 end with the score of the first query (rows 0-7), lanes 32-47
// with the second (rows 8-15).  The head weights are >= 0, so every score is
// >= +0 (or -inf where masked).
__device__ __forceinline__ float head_part(f32x4 acc, const float w4[4]) {
  float s = w4[0] * relu(acc[0]);
  s = fmaf(w4[1], relu(acc[1]), s);
  s = fmaf(w4[2], relu(acc[2]), s);
  return fmaf(w4[3], relu(acc[3]), s);
}
__device__ __forceinline__ float head_sum(f32x4 acc, const float w4[4]) {
  return sum_xor16(head_part(acc, w4));
}

// Head sums of two accumulator fragments (query pairs A and B) with one
// cross-lane swap: v_permlane16_swap exchanges the odd 16-lane rows of the
// first operand with the even rows of the second, so the sum of the two
// results holds, in 16-lane rows 0..3, the scores of A's first query, B's
// first query, A's second query and B's second query.  Every score is the
// same two partial sums added as in head_sum, so the bits are the same.
__device__ __forceinline__ float head_sum_pair(f32x4 a, const float wa[4], f32x4 b, const float wb[4]) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(head_part(a, wa)),
                                                  __float_as_uint(head_part(b, wb)), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max over aligned groups of 8 lanes for scores (>= +0 or -inf): on that
// set the float order is the int32 order of the bit patterns, so the DPP
// steps are integer maxes.
// (Every lane has a source lane under these controls, so a plain DPP move,
// which the compiler folds into the max as its DPP operand, is enough.)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true); }
__device__ __forceinline__ float score_max8(float v) {
  int b = __float_as_int(v), o;
  o = dpp_i<0xB1>(b); b = b > o ? b : o;
  o = dpp_i<0x4E>(b); b = b > o ? b : o;
  o = dpp_i<0x141>(b); b = b > o ? b : o;
  return __int_as_float(b);
}

// Store one fragment's scores / block maxima.  `v` is the lane's score or
// -inf; only lanes with (lane & 16) == 0 own an output.
__device__ __forceinline__ void store_frag(float v, int64_t q, int64_t col, int64_t ncols,
                                           int64_t nblk, float* scores, float* block_max, int lane,
                                           bool owner) {
  if (scores && owner && col < ncols) scores[q * ncols + col] = v;
  if (block_max) {
    const float m = score_max8(v);
    int64_t blk = col >> 3;
    if (owner && (lane & 7) == 0 && blk < nblk) block_max[q * nblk + blk] = m;
  }
}

}  // namespace idxf
}  // namespace csa

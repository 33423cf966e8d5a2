// Sparse multi-query attention over the selected MXFP4 entries plus the
// FP8 sliding window.
//
// P3 §02: the selected Top-K entries are used for attention; one shared latent
// serves all query heads (fewer KV heads).  P3 §03: the FP4 cache is
// dequantized before attention (no FP4 matmul), the SWA window stays FP8 and
// covers n_win = 128 tokens.
//
// Work item = (query, split of its key slots); one wave per work item.  Key
// slots 0..k-1 are the selected entries, slots k..k+127 the window tokens
// p-127..p.  Per 16-slot tile:
//   1. each lane loads 128 channels of one key (FP4 codes + E4M3 scales, or
//      E4M3 window bytes) and dequantizes them in registers to fp16 (exact);
//   2. S^T = K Q^T on the fp16 matrix cores (16 x v_mfma 16x16x32), keys as
//      rows so that the result is already the A operand of P V;
//   3. online softmax in float32 (log2 domain);
//   4. the fp16 tile goes through LDS so that each lane can gather 4 keys of
//      one channel for the B operand of P V (32 x v_mfma 16x16x16).  The
//      output channel of N-tile n in lane column c is 32 c + n, so every lane
//      reads 64 contiguous bytes per key.
// With several splits per query the partial (O, max, sum) triples are
// combined by attn_combine_kernel.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int AT_TILE = 16;
constexpr int AT_PITCH = D * 2 + 16;   // bytes per LDS key row (fp16 + pad)

struct AttnArgs {
  const float* q;
  const int32_t* q_pos;
  int64_t q_per_seq;
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t kv_rows;
  const int32_t* idx;
  int32_t k;
  const uint8_t* win;
  int64_t win_cap;
  float c_log2;          // sm_scale * log2(e)
  float* out;
  float* part_o;         // [Q, n_splits, 16, 512] (n_splits > 1)
  float* part_ml;        // [Q, n_splits, 2, 16]
  int n_splits;
  int tiles_per_split;
};

__global__ __launch_bounds__(64) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[AT_TILE * AT_PITCH];
  const int lane = threadIdx.x;
  const int j = lane & 15;      // key slot in the tile (loads), head (softmax, Q)
  const int g = lane >> 4;      // 128-channel quarter (loads), key group of 4 (S, P)
  const int64_t qi = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t seq = qi / a.q_per_seq;
  const int32_t p = a.q_pos[qi];
  const int n_slots = a.k + NWIN;
  const int n_tiles = (n_slots + AT_TILE - 1) / AT_TILE;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  t_end = t_end < n_tiles ? t_end : n_tiles;

  // Q: head j, channels 128 g .. 128 g + 127, rounded to fp16
  f16x2 qf[64];
  {
    const float4* src = reinterpret_cast<const float4*>(a.q + (qi * HEADS + j) * D + 128 * g);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float4 f = src[i];
      qf[2 * i] = f16x2{(_Float16)f.x, (_Float16)f.y};
      qf[2 * i + 1] = f16x2{(_Float16)f.z, (_Float16)f.w};
    }
  }
  f32x4 acc_o[32];
#pragma unroll
  for (int n = 0; n < 32; ++n) acc_o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const uint8_t* codes_seq = a.codes + seq * a.kv_rows * CODE_BYTES;
  const uint8_t* scales_seq = a.scales + seq * a.kv_rows * SCALE_BYTES;
  const uint8_t* win_seq = a.win + seq * a.win_cap * D;

  for (int t = t_begin; t < t_end; ++t) {
    // ---- 1. load + dequantize this lane's key quarter --------------------
    const int slot = t * AT_TILE + j;
    bool valid = false;
    f16x2 kf[64];
    if (slot < a.k) {
      int32_t id = a.idx[qi * a.k + slot];
      valid = id >= 0 && id < a.kv_rows;
      uint4 cw[4] = {};
      uint2 sw = {0u, 0u};
      if (valid) {
        const uint4* cp = reinterpret_cast<const uint4*>(codes_seq + (int64_t)id * CODE_BYTES + 64 * g);
        cw[0] = cp[0]; cw[1] = cp[1]; cw[2] = cp[2]; cw[3] = cp[3];
        sw = *reinterpret_cast<const uint2*>(scales_seq + (int64_t)id * SCALE_BYTES + 8 * g);
      }
      f16x2 s01 = fp8x2_to_f16<0>(sw.x), s23 = fp8x2_to_f16<1>(sw.x);
      f16x2 s45 = fp8x2_to_f16<0>(sw.y), s67 = fp8x2_to_f16<1>(sw.y);
      _Float16 sc[8] = {s01[0], s01[1], s23[0], s23[1], s45[0], s45[1], s67[0], s67[1]};
      const uint32_t words[16] = {cw[0].x, cw[0].y, cw[0].z, cw[0].w, cw[1].x, cw[1].y, cw[1].z, cw[1].w,
                                  cw[2].x, cw[2].y, cw[2].z, cw[2].w, cw[3].x, cw[3].y, cw[3].z, cw[3].w};
#pragma unroll
      for (int d = 0; d < 16; ++d) {          // dword d: channels 8d .. 8d+7 of the quarter
        f16x2 s2 = f16x2{sc[d >> 1], sc[d >> 1]};
        kf[4 * d + 0] = fp4x2_to_f16<0>(words[d]) * s2;
        kf[4 * d + 1] = fp4x2_to_f16<1>(words[d]) * s2;
        kf[4 * d + 2] = fp4x2_to_f16<2>(words[d]) * s2;
        kf[4 * d + 3] = fp4x2_to_f16<3>(words[d]) * s2;
      }
    } else {
      const int w = slot - a.k;
      const int64_t wp = (int64_t)p - (NWIN - 1) + w;
      valid = w < NWIN && wp >= 0;
      uint4 ww[8] = {};
      if (valid) {
        const uint4* wptr = reinterpret_cast<const uint4*>(win_seq + (wp % a.win_cap) * D + 128 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) ww[i] = wptr[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w4[4] = {ww[i].x, ww[i].y, ww[i].z, ww[i].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kf[8 * i + 2 * u] = fp8x2_to_f16<0>(w4[u]);
          kf[8 * i + 2 * u + 1] = fp8x2_to_f16<1>(w4[u]);
        }
      }
    }
    const uint32_t vmask = (uint32_t)(__ballot(valid) & 0xFFFFull);

    // ---- 2. S^T = K Q^T ---------------------------------------------------
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      f16x8 av = {kf[4 * s][0], kf[4 * s][1], kf[4 * s + 1][0], kf[4 * s + 1][1],
                  kf[4 * s + 2][0], kf[4 * s + 2][1], kf[4 * s + 3][0], kf[4 * s + 3][1]};
      f16x8 bv = {qf[4 * s][0], qf[4 * s][1], qf[4 * s + 1][0], qf[4 * s + 1][1],
                  qf[4 * s + 2][0], qf[4 * s + 2][1], qf[4 * s + 3][0], qf[4 * s + 3][1]};
      sacc = mfma_f16_16x16x32(av, bv, sacc);
    }

    // ---- 3. online softmax (lane: keys 4g+r, head j) ------------------------
    float x[4];
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bool ok = (vmask >> (4 * g + r)) & 1u;
      x[r] = ok ? sacc[r] * a.c_log2 : -__builtin_huge_valf();
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == -__builtin_huge_valf()) ? 0.f : m_new;
    const float alpha = (m_run == -__builtin_huge_valf()) ? 0.f : exp2f(m_run - base);
    float pr[4], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = exp2f(x[r] - base);
      psum += pr[r];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale O rows (heads 4g + r) when a head's max moved
    if (__ballot(alpha != 1.0f)) {
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        acc_o[n][0] *= al[0]; acc_o[n][1] *= al[1];
        acc_o[n][2] *= al[2]; acc_o[n][3] *= al[3];
      }
    }
    const f16x4 pa = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};

    // ---- 4. P V through LDS ---------------------------------------------------
    __syncthreads();   // previous tile's LDS reads are done
    {
      uint4* dst = reinterpret_cast<uint4*>(lds + j * AT_PITCH + 256 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dst[i] = make_uint4(f16x2_bits(kf[4 * i]), f16x2_bits(kf[4 * i + 1]), f16x2_bits(kf[4 * i + 2]),
                            f16x2_bits(kf[4 * i + 3]));
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {             // channels 32 j + 8c .. +8
      uint4 v[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        v[kk] = *reinterpret_cast<const uint4*>(lds + (4 * g + kk) * AT_PITCH + 64 * j + 16 * c);
      const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
      const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
      const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
      const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // channel pair (2i, 2i+1) of the 8: N-tiles n = 8c + 2i and 8c + 2i + 1
        uint32_t lo01 = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);
        uint32_t lo23 = __builtin_amdgcn_perm(w3[i], w2[i], 0x05040100u);
        uint32_t hi01 = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);
        uint32_t hi23 = __builtin_amdgcn_perm(w3[i], w2[i], 0x07060302u);
        f16x2 a0 = bits_f16x2(lo01), a1 = bits_f16x2(lo23);
        f16x2 b0 = bits_f16x2(hi01), b1 = bits_f16x2(hi23);
        f16x4 blo = {a0[0], a0[1], a1[0], a1[1]};
        f16x4 bhi = {b0[0], b0[1], b1[0], b1[1]};
        acc_o[8 * c + 2 * i] = mfma_f16_16x16x16(pa, blo, acc_o[8 * c + 2 * i]);
        acc_o[8 * c + 2 * i + 1] = mfma_f16_16x16x16(pa, bhi, acc_o[8 * c + 2 * i + 1]);
      }
    }
  }

  // ---- epilogue: lane holds O[head 4g + r][channel 32 j + n] ---------------
  if (a.n_splits == 1) {
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float l = __shfl(l_run, 4 * g + r);
      inv[r] = l > 0.f ? 1.0f / l : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(a.out + (qi * HEADS + 4 * g + r) * D + 32 * j);
#pragma unroll
      for (int n4 = 0; n4 < 8; ++n4)
        dst[n4] = make_float4(acc_o[4 * n4][r] * inv[r], acc_o[4 * n4 + 1][r] * inv[r],
                              acc_o[4 * n4 + 2][r] * inv[r], acc_o[4 * n4 + 3][r] * inv[r]);
    }
  } else {
    const int64_t ps = qi * a.n_splits + split;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(a.part_o + (ps * HEADS + 4 * g + r) * D + 32 * j);
#pragma unroll
      for (int n4 = 0; n4 < 8; ++n4)
        dst[n4] = make_float4(acc_o[4 * n4][r], acc_o[4 * n4 + 1][r], acc_o[4 * n4 + 2][r],
                              acc_o[4 * n4 + 3][r]);
    }
    if (lane < 16) {
      a.part_ml[(ps * 2 + 0) * HEADS + j] = m_run;
      a.part_ml[(ps * 2 + 1) * HEADS + j] = l_run;
    }
  }
}

// out[q, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.  One block of
// 128 threads per (query, head), 4 channels per thread.
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, float* __restrict__ out) {
  const int64_t qi = blockIdx.y;
  const int h = blockIdx.x;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_ml[((qi * n_splits + s) * 2) * HEADS + h]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t ps = qi * n_splits + s;
    float m = part_ml[(ps * 2) * HEADS + h];
    float l = part_ml[(ps * 2 + 1) * HEADS + h];
    float wgt = (m == -__builtin_huge_valf()) ? 0.f : exp2f(m - M);
    L = fmaf(wgt, l, L);
    float4 o = reinterpret_cast<const float4*>(part_o + (ps * HEADS + h) * D)[threadIdx.x];
    acc.x = fmaf(wgt, o.x, acc.x); acc.y = fmaf(wgt, o.y, acc.y);
    acc.z = fmaf(wgt, o.z, acc.z); acc.w = fmaf(wgt, o.w, acc.w);
  }
  float inv = L > 0.f ? 1.0f / L : 0.f;
  reinterpret_cast<float4*>(out + (qi * HEADS + h) * D)[threadIdx.x] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

namespace {
void attn_plan(int64_t Q, int32_t k, int* n_splits, int* tiles_per_split) {
  int n_tiles = (k + NWIN + AT_TILE - 1) / AT_TILE;
  int64_t want = Q >= 1024 ? 1 : (1024 + Q - 1) / Q;     // aim at ~1024 waves
  int max_split = (n_tiles + 1) / 2;                      // at least 2 tiles per split
  int s = (int)(want < max_split ? want : max_split);
  s = s < 1 ? 1 : s;
  int tps = (n_tiles + s - 1) / s;
  *tiles_per_split = tps;
  *n_splits = (n_tiles + tps - 1) / tps;
}
}  // namespace

size_t attn_workspace_bytes(int64_t Q, int32_t k) {
  int ns, tps;
  attn_plan(Q, k, &ns, &tps);
  if (ns <= 1) return 0;
  size_t po = (size_t)Q * ns * HEADS * D * sizeof(float);
  size_t pm = (size_t)Q * ns * 2 * HEADS * sizeof(float);
  return po + pm;
}

hipError_t launch_sparse_attn(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                              const uint8_t* codes, const uint8_t* scales, int64_t kv_rows,
                              const int32_t* idx, int32_t k, const uint8_t* win, int64_t win_cap,
                              float sm_scale, float* out, void* ws, hipStream_t st) {
  int64_t Q = n_seq * q_per_seq;
  if (Q == 0) return hipSuccess;
  AttnArgs a;
  a.q = q; a.q_pos = q_pos; a.q_per_seq = q_per_seq;
  a.codes = codes; a.scales = scales; a.kv_rows = kv_rows;
  a.idx = idx; a.k = k; a.win = win; a.win_cap = win_cap;
  a.c_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  attn_plan(Q, k, &a.n_splits, &a.tiles_per_split);
  a.part_o = nullptr; a.part_ml = nullptr;
  if (a.n_splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)Q * a.n_splits * HEADS * D;
  }
  hipLaunchKernelGGL(attn_kernel, dim3(a.n_splits, (unsigned)Q), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(HEADS, (unsigned)Q), dim3(128), 0, st, a.part_o, a.part_ml,
                     a.n_splits, out);
  return hipGetLastError();
}

}  // namespace csa

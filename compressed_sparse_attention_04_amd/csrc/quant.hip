// MXFP4 store path: quantize / dequantize, window append, and the fused
// compress (4 tokens -> 1 entry) + RMSNorm + RoPE + quantize chain.
//
// "DeepSeek-V4.1 架构解析" §02 (sequence compression), the DeepSeek V4 overview page §2.1 (4:1), "DeepSeek-V4.1 架构解析" §03 (E2M1 values with an
// E4M3 scale per 16 channels, RMSNorm before, quantize after RoPE; SWA KV in
// FP8).
#include "common.h"
#include "kernels.h"

namespace csa {

// ---------------------------------------------------------------------------
// Quantize: 16 lanes per entry, 32 channels (two scale groups) per lane.
// Each lane stores its 16 code bytes with one 16-byte store (an entry's 256
// code bytes are one contiguous 256-byte run) and its two scale bytes.
__device__ __forceinline__ void quantize32_store(const float* v, uint8_t* codes_row,
                                                 uint8_t* scales_row, int lane16) {
  uint32_t c0[2], c1[2];
  uint32_t s0 = mxfp4_group(v, c0);
  uint32_t s1 = mxfp4_group(v + 16, c1);
  uint4 cw = make_uint4(c0[0], c0[1], c1[0], c1[1]);
  *reinterpret_cast<uint4*>(codes_row + 16 * lane16) = cw;
  *reinterpret_cast<uint16_t*>(scales_row + 2 * lane16) = (uint16_t)(s0 | (s1 << 8));
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ e, int64_t n,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t entry = t >> 4;
  int lane16 = (int)(t & 15);
  if (entry >= n) return;
  const float4* src = reinterpret_cast<const float4*>(e + entry * D + 32 * lane16);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 f = src[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  quantize32_store(v, codes + entry * CODE_BYTES, scales + entry * SCALE_BYTES, lane16);
}

__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         int64_t n, float* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t entry = t >> 4;
  int lane16 = (int)(t & 15);
  if (entry >= n) return;
  uint4 cw = *reinterpret_cast<const uint4*>(codes + entry * CODE_BYTES + 16 * lane16);
  uint16_t sw = *reinterpret_cast<const uint16_t*>(scales + entry * SCALE_BYTES + 2 * lane16);
  float s0 = e4m3_code_value(sw & 0x7Fu), s1 = e4m3_code_value((sw >> 8) & 0x7Fu);
  uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
  float4* dst = reinterpret_cast<float4*>(out + entry * D + 32 * lane16);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = i < 4 ? s0 : s1;
    uint32_t word = w[i >> 1] >> (16 * (i & 1));
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t c = (word >> (4 * j)) & 0xFu;
      float m = e2m1_value(c) * s;
      f[j] = (c & 8u) ? -m : m;
    }
    dst[i] = make_float4(f[0], f[1], f[2], f[3]);
  }
}

// ---------------------------------------------------------------------------
// Window append: 32 lanes per token, 16 channels per lane, one 16-byte store.
// Thread t of the launch (t = 256 block + thread) takes lane t % 32 of token
// t / 32.
__device__ __forceinline__ void window_append_thread(const WindowAppendArgs& a, int64_t t) {
  int64_t tok = t >> 5;
  int lane = (int)(t & 31);
  if (tok >= a.n_seq * a.n_tok) return;
  int64_t s = tok / a.n_tok, i = tok % a.n_tok;
  int64_t p = (int64_t)a.pos0[s] + i;
  if (p < 0) return;
  const float4* src = reinterpret_cast<const float4*>(a.x + s * a.x_seq_stride + i * D + 16 * lane);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float4 f = src[k];
    w[k] = e4m3_encode(f.x) | (e4m3_encode(f.y) << 8) | (e4m3_encode(f.z) << 16) |
           (e4m3_encode(f.w) << 24);
  }
  uint8_t* dst = a.win + (s * a.win_cap + p % a.win_cap) * D + 16 * lane;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void window_append_kernel(WindowAppendArgs a) {
  window_append_thread(a, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

int64_t window_append_blocks(const WindowAppendArgs& a) { return (a.n_seq * a.n_tok * 32 + 255) / 256; }

// ---------------------------------------------------------------------------
// Window rebuild from the latest tokens: 32 lanes per ring row, 16 channels
// per lane.  Row j of ring r holds the token at the latest position t <= p
// with t = j (mod win_cap) when that token is one of the n_tok given
// (t >= p - n_tok + 1, t >= 0), else zeros.
__global__ __launch_bounds__(256) void window_rebuild_kernel(const float* __restrict__ x,
                                                             int64_t n_ring, int64_t n_tok,
                                                             int64_t x_ring_stride,
                                                             const int32_t* __restrict__ p_last,
                                                             uint8_t* __restrict__ win,
                                                             int64_t win_cap) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t >> 5;
  const int lane = (int)(t & 31);
  if (row >= n_ring * win_cap) return;
  const int64_t r = row / win_cap, j = row % win_cap;
  const int64_t p = p_last[r];
  const int64_t pos = p - (((p - j) % win_cap) + win_cap) % win_cap;   // latest position <= p in row j
  const int64_t i = pos - (p - n_tok + 1);                                // its index among the tokens
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (pos >= 0 && i >= 0) {
    const float4* src = reinterpret_cast<const float4*>(x + r * x_ring_stride + i * D + 16 * lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 f = src[k];
      w[k] = e4m3_encode(f.x) | (e4m3_encode(f.y) << 8) | (e4m3_encode(f.z) << 16) |
             (e4m3_encode(f.w) << 24);
    }
  }
  uint8_t* dst = win + row * D + 16 * lane;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// Compression GEMM on the fp64 matrix cores: Y[i, o] = sum_k Xc[i, k] Wc[o, k]
// with Xc[i] = the 4 token rows of entry i (2048 contiguous floats) and
// Wc[o, i*512 + c] = W_i[o, c].  Every fp32 x fp32 product is exact in fp64,
// and the chain (GEMM, RMSNorm, RoPE) stays in fp64 until the quantizer input
// is rounded to fp32 once; so that input is the correctly rounded value of the
// exact result except within ~1e-13 (relative) of an fp32 rounding boundary,
// and the stored bytes do not depend on the summation order.
// Tile 32 entries x 64 outputs, k-chunks of 32; optional split-K over
// blockIdx.z writes partial sums to ypart[z].
constexpr int CG_BM = 32, CG_BN = 64, CG_BK = 32, CG_PITCH = CG_BK + 1;

__global__ __launch_bounds__(256) void compress_gemm_kernel(const float* __restrict__ x,
                                                            int64_t n_seq, int64_t n_per_seq,
                                                            int64_t x_seq_stride,
                                                            const float* __restrict__ w,
                                                            double* __restrict__ ypart,
                                                            int k_per_split) {
  __shared__ float As[CG_BM][CG_PITCH];
  __shared__ float Bs[CG_BN][CG_PITCH];
  const int64_t n = n_seq * n_per_seq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int o0 = blockIdx.x * CG_BN;
  const int64_t r0 = (int64_t)blockIdx.y * CG_BM;
  const int kbeg = blockIdx.z * k_per_split;
  const int kend = kbeg + k_per_split;
  // A loads: one float4 per thread (32 rows x 8 float4)
  const int a_row = tid >> 3, a_k4 = (tid & 7) * 4;
  const int64_t a_entry = r0 + a_row;
  const float* a_src = nullptr;
  if (a_entry < n) {
    int64_t s = a_entry / n_per_seq, r = a_entry % n_per_seq;
    a_src = x + s * x_seq_stride + r * (4 * D);
  }
  const int wr = (wave >> 1) * 16;          // wave's row offset in the tile
  const int wc = (wave & 1) * 32;           // wave's column offset
  f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  // chunk k0's A and B values in registers; the next chunk's loads are
  // issued before this chunk's products, so they overlap them
  float4 av, bv[2];
  auto load_chunk = [&](int k0) {
    av = a_src ? *reinterpret_cast<const float4*>(a_src + k0 + a_k4) : make_float4(0.f, 0.f, 0.f, 0.f);
    const int ti = k0 / D, c0 = k0 % D;     // token slot and channel of this chunk
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int idx = tid + 256 * u;
      int row = idx >> 3, k4 = (idx & 7) * 4;
      bv[u] = *reinterpret_cast<const float4*>(w + (int64_t)ti * D * D + (int64_t)(o0 + row) * D +
                                               c0 + k4);
    }
  };
  load_chunk(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += CG_BK) {
    __syncthreads();   // the previous chunk's products have read the tiles
    As[a_row][a_k4] = av.x; As[a_row][a_k4 + 1] = av.y;
    As[a_row][a_k4 + 2] = av.z; As[a_row][a_k4 + 3] = av.w;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int idx = tid + 256 * u;
      int row = idx >> 3, k4 = (idx & 7) * 4;
      Bs[row][k4] = bv[u].x; Bs[row][k4 + 1] = bv[u].y;
      Bs[row][k4 + 2] = bv[u].z; Bs[row][k4 + 3] = bv[u].w;
    }
    __syncthreads();
    if (k0 + CG_BK < kend) load_chunk(k0 + CG_BK);
#pragma unroll
    for (int kk = 0; kk < CG_BK; kk += 4) {
      double a = As[wr + (lane & 15)][kk + (lane >> 4)];
      double b0 = Bs[wc + (lane & 15)][kk + (lane >> 4)];
      double b1 = Bs[wc + 16 + (lane & 15)][kk + (lane >> 4)];
      acc0 = mfma_f64_16x16x4(a, b0, acc0);
      acc1 = mfma_f64_16x16x4(a, b1, acc1);
    }
  }
  double* yp = ypart + (int64_t)blockIdx.z * n * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int64_t row = r0 + wr + (lane >> 4) + 4 * r;      // fp64 16x16x4 result layout
    if (row < n) {
      yp[row * D + o0 + wc + (lane & 15)] = acc0[r];
      yp[row * D + o0 + wc + 16 + (lane & 15)] = acc1[r];
    }
  }
}

// RMSNorm + RoPE (fp64) + quantize + packed store.  One 256-thread block per
// entry, channels 2t and 2t+1 per thread (one RoPE pair).  The split-K
// partials are loaded together and summed in a fixed order; a 16-channel scale
// group is 8 adjacent threads.  The packed row is assembled in LDS and stored
// with 16-byte stores (codes: 16 lanes x 16 B, scales: 2 lanes x 16 B).
constexpr int CE_MAX_SPLIT = 16;

__device__ __forceinline__ void compress_epilogue_entry(
    int64_t entry, const double* __restrict__ ypart, int n_split, int64_t n_seq, int64_t n_per_seq,
    const float* __restrict__ rope_cs, int rope_dim, float eps, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t out_seq_stride, float* __restrict__ e_out) {
  __shared__ double red[4];
  __shared__ __attribute__((aligned(16))) uint8_t row_codes[CODE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t row_scales[SCALE_BYTES];
  const int64_t n = n_seq * n_per_seq;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  double2 part[CE_MAX_SPLIT];
#pragma unroll
  for (int z = 0; z < CE_MAX_SPLIT; ++z)
    if (z < n_split) part[z] = reinterpret_cast<const double2*>(ypart + ((int64_t)z * n + entry) * D)[t];
  double y0 = 0.0, y1 = 0.0;
#pragma unroll
  for (int z = 0; z < CE_MAX_SPLIT; ++z)
    if (z < n_split) { y0 += part[z].x; y1 += part[z].y; }
  double ss = fma(y0, y0, y1 * y1);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const double inv = 1.0 / sqrt(ss * (1.0 / (double)D) + (double)eps);
  y0 *= inv;
  y1 *= inv;
  const int c = 2 * t;
  if (rope_dim > 0 && c >= D - rope_dim) {
    const float* cs = rope_cs + entry * (int64_t)rope_dim + 2 * ((c - (D - rope_dim)) >> 1);
    const double cc = cs[0], sn = cs[1];
    const double x0 = y0, x1 = y1;
    y0 = x0 * cc - x1 * sn;
    y1 = x0 * sn + x1 * cc;
  }
  const float v0 = (float)y0, v1 = (float)y1;
  if (e_out) reinterpret_cast<float2*>(e_out + entry * D)[t] = make_float2(v0, v1);
  // scale of the 16-channel group held by threads 8k .. 8k+7
  float amax = fmaxf(fabsf(v0), fabsf(v1));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const uint32_t sc = e4m3_scale_code(amax);
  const float sv = e4m3_code_value(sc);
  row_codes[t] = (uint8_t)(e2m1_code(v0, sv, sc) | (e2m1_code(v1, sv, sc) << 4));
  if ((t & 7) == 0) row_scales[t >> 3] = (uint8_t)sc;
  __syncthreads();
  const int64_t s = entry / n_per_seq, r = entry % n_per_seq;
  const int64_t row = s * out_seq_stride + r;
  if (t < 16)
    reinterpret_cast<uint4*>(codes + row * CODE_BYTES)[t] = reinterpret_cast<const uint4*>(row_codes)[t];
  else if (t < 18)
    reinterpret_cast<uint4*>(scales + row * SCALE_BYTES)[t - 16] =
        reinterpret_cast<const uint4*>(row_scales)[t - 16];
}

__global__ __launch_bounds__(256) void compress_epilogue_kernel(
    const double* __restrict__ ypart, int n_split, int64_t n_seq, int64_t n_per_seq,
    const float* __restrict__ rope_cs, int rope_dim, float eps, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t out_seq_stride, float* __restrict__ e_out) {
  compress_epilogue_entry(blockIdx.x, ypart, n_split, n_seq, n_per_seq, rope_cs, rope_dim, eps, codes, scales,
                          out_seq_stride, e_out);
}

// The epilogue and a window append in one launch (independent outputs):
// blocks below n finish entries, the blocks after them append tokens.
__global__ __launch_bounds__(256) void compress_epilogue_append_kernel(
    const double* __restrict__ ypart, int n_split, int64_t n_seq, int64_t n_per_seq,
    const float* __restrict__ rope_cs, int rope_dim, float eps, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t out_seq_stride, float* __restrict__ e_out, WindowAppendArgs ap) {
  const int64_t n = n_seq * n_per_seq;
  if ((int64_t)blockIdx.x >= n) {   // block-uniform, before any barrier
    window_append_thread(ap, ((int64_t)blockIdx.x - n) * 256 + threadIdx.x);
    return;
  }
  compress_epilogue_entry(blockIdx.x, ypart, n_split, n_seq, n_per_seq, rope_cs, rope_dim, eps, codes, scales,
                          out_seq_stride, e_out);
}

// ------------------------------------------------------------- launchers --
hipError_t launch_quantize(const float* e, int64_t n, uint8_t* codes, uint8_t* scales,
                           hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n * 16 + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, e, n, codes, scales);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out,
                             hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n * 16 + 255) / 256;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, scales, n, out);
  return hipGetLastError();
}

hipError_t launch_window_append(const float* x, int64_t n_seq, int64_t n_tok, int64_t x_seq_stride,
                                const int32_t* pos0, uint8_t* win, int64_t win_cap, hipStream_t st) {
  const WindowAppendArgs a{x, n_seq, n_tok, x_seq_stride, pos0, win, win_cap};
  if (n_seq * n_tok == 0) return hipSuccess;
  hipLaunchKernelGGL(window_append_kernel, dim3((unsigned)window_append_blocks(a)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_window_rebuild(const float* x, int64_t n_ring, int64_t n_tok, int64_t x_ring_stride,
                                 const int32_t* p_last, uint8_t* win, int64_t win_cap, hipStream_t st) {
  const int64_t rows = n_ring * win_cap;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * 32 + 255) / 256;
  hipLaunchKernelGGL(window_rebuild_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n_ring, n_tok,
                     x_ring_stride, p_last, win, win_cap);
  return hipGetLastError();
}

int compress_split_k(int64_t n) {
  int64_t tiles = (int64_t)(D / CG_BN) * ((n + CG_BM - 1) / CG_BM);
  int split = 1;
  // spread small batches over more blocks: K = 2048 split into up to 16 parts
  while (split < 16 && tiles * split < 512) split *= 2;
  return split;
}

size_t compress_workspace_bytes(int64_t n) {
  return (size_t)compress_split_k(n) * (size_t)n * D * sizeof(double);
}

hipError_t launch_compress_quant(const float* x, int64_t n_seq, int64_t n_per_seq,
                                 int64_t x_seq_stride, const float* w, const float* rope_cs,
                                 int rope_dim, float eps, uint8_t* codes, uint8_t* scales,
                                 int64_t out_seq_stride, float* e_out, void* ws, hipStream_t st,
                                 const WindowAppendArgs* append) {
  int64_t n = n_seq * n_per_seq;
  const int64_t app_blocks = (append && append->n_seq * append->n_tok > 0) ? window_append_blocks(*append) : 0;
  if (n == 0) {
    if (app_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(window_append_kernel, dim3((unsigned)app_blocks), dim3(256), 0, st, *append);
    return hipGetLastError();
  }
  int split = compress_split_k(n);
  double* ypart = reinterpret_cast<double*>(ws);
  dim3 grid(D / CG_BN, (unsigned)((n + CG_BM - 1) / CG_BM), split);
  hipLaunchKernelGGL(compress_gemm_kernel, grid, dim3(256), 0, st, x, n_seq, n_per_seq, x_seq_stride,
                     w, ypart, (4 * D) / split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (app_blocks > 0)
    hipLaunchKernelGGL(compress_epilogue_append_kernel, dim3((unsigned)(n + app_blocks)), dim3(256), 0, st, ypart,
                       split, n_seq, n_per_seq, rope_cs, rope_dim, eps, codes, scales, out_seq_stride, e_out,
                       *append);
  else
    hipLaunchKernelGGL(compress_epilogue_kernel, dim3((unsigned)n), dim3(256), 0, st, ypart, split,
                       n_seq, n_per_seq, rope_cs, rope_dim, eps, codes, scales, out_seq_stride, e_out);
  return hipGetLastError();
}

}  // namespace csa

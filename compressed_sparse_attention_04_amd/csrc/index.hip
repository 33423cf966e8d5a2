// Indexer scoring on the FP8 matrix cores.
//
// P3 §02: Full layers score every causally visible position; Reindex layers
// rescore with their own indexer query, inside the hierarchical pool.
// score_j = sum_h w_h * ReLU(q_h . k_j), 8 heads x 128 dims, E4M3 operands.
//
// One v_mfma 16x16x128 (fp8) contracts a 16-row A fragment (8 heads of one
// query, or 8 heads each of two queries) against 16 indexer keys: the whole
// 128-wide head dimension is a single instruction.  The epilogue applies
// ReLU and the head weights on the accumulator (lane l holds rows
// 4*(l/16)+r, column l%16), folds the two 16-lane halves that hold the 8
// heads of a query, and optionally reduces 8 adjacent columns to a block max.
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

// A-fragment register block of one lane: 32 fp8 bytes of one (query, head)
// row: bytes 32 * (lane / 16) .. +32.  Rows whose query is absent are zero.
__device__ __forceinline__ i32x8 load_qfrag(const uint8_t* q_fp8, int64_t q, int head, bool live,
                                            int lane) {
  i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
    const uint4* p = reinterpret_cast<const uint4*>(q_fp8 + (q * IH + head) * ID + 32 * (lane >> 4));
    uint4 u0 = p[0], u1 = p[1];
    a[0] = u0.x; a[1] = u0.y; a[2] = u0.z; a[3] = u0.w;
    a[4] = u1.x; a[5] = u1.y; a[6] = u1.z; a[7] = u1.w;
  }
  return a;
}

// B fragment: lane l loads bytes 32 * (l / 16) .. +32 of key row `e`.
__device__ __forceinline__ i32x8 load_kfrag(const uint8_t* krow_base, int64_t e, bool live, int lane) {
  i32x8 b = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
    const uint4* p = reinterpret_cast<const uint4*>(krow_base + e * ID + 32 * (lane >> 4));
    uint4 u0 = p[0], u1 = p[1];
    b[0] = u0.x; b[1] = u0.y; b[2] = u0.z; b[3] = u0.w;
    b[4] = u1.x; b[5] = u1.y; b[6] = u1.z; b[7] = u1.w;
  }
  return b;
}

// Weighted ReLU head sum of one accumulator fragment; lanes 0-15 end with the
// score of the first query (rows 0-7), lanes 32-47 with the second (rows 8-15).
__device__ __forceinline__ float head_sum(f32x4 acc, const float w4[4]) {
  float s = w4[0] * fmaxf(acc[0], 0.f);
  s = fmaf(w4[1], fmaxf(acc[1], 0.f), s);
  s = fmaf(w4[2], fmaxf(acc[2], 0.f), s);
  s = fmaf(w4[3], fmaxf(acc[3], 0.f), s);
  return s + __shfl_xor(s, 16);
}

// Store one fragment's scores / block maxima.  `v` is the lane's score or
// -inf; only lanes with (lane & 16) == 0 own an output.
__device__ __forceinline__ void store_frag(float v, int64_t q, int64_t col, int64_t ncols,
                                           int64_t nblk, float* scores, float* block_max, int lane,
                                           bool owner) {
  if (scores && owner && col < ncols) scores[q * ncols + col] = v;
  if (block_max) {
    float m = fmaxf(v, __shfl_xor(v, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    int64_t blk = col >> 3;
    if (owner && (lane & 7) == 0 && blk < nblk) block_max[q * nblk + blk] = m;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// One query per block (decode, and every pooled call): the block covers
// SQ_COLS columns, each of its 4 waves SQ_COLS / 4 of them, 16 per MFMA.
constexpr int SQ_COLS = 1024;
constexpr int SQ_UNROLL = 4;

template <bool POOLED>
__global__ __launch_bounds__(256) void score_query_kernel(ScoreArgs a, int64_t ncols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = blockIdx.y;
  const int64_t seq = q / a.q_per_seq;
  const int nv_pos = visible_count(a.q_pos[q]);
  const int64_t nv = nv_pos < a.n_entries ? nv_pos : a.n_entries;
  const int row = lane & 15;
  const i32x8 afrag = load_qfrag(a.q_fp8, q, row, row < IH, lane);
  float w4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int h = 4 * (lane >> 4) + r;
    w4[r] = (lane < 32) ? a.w[q * IH + h] : 0.f;
  }
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  const int64_t nblk = (ncols + 7) >> 3;
  const int64_t c_wave = (int64_t)blockIdx.x * SQ_COLS + wave * (SQ_COLS / 4);
  for (int f0 = 0; f0 < SQ_COLS / 4 / 16; f0 += SQ_UNROLL) {
    i32x8 b[SQ_UNROLL];
    bool valid[SQ_UNROLL];
#pragma unroll
    for (int u = 0; u < SQ_UNROLL; ++u) {
      int64_t col = c_wave + 16 * (f0 + u) + (lane & 15);
      int64_t e = col;
      bool ok = col < ncols;
      if (POOLED && ok) {
        int32_t blk = a.pool[q * a.n_pool_blocks + (col >> 3)];
        ok = blk >= 0;
        e = 8 * (int64_t)blk + (col & 7);
      }
      ok = ok && e < nv;
      valid[u] = ok;
      b[u] = load_kfrag(kbase, e, ok, lane);
    }
#pragma unroll
    for (int u = 0; u < SQ_UNROLL; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_f8_16x16x128(afrag, b[u], acc);
      float s = head_sum(acc, w4);
      int64_t col = c_wave + 16 * (f0 + u) + (lane & 15);
      float v = valid[u] ? s : -__builtin_huge_valf();
      store_frag(v, q, col, ncols, nblk, a.scores, POOLED ? nullptr : a.block_max, lane, lane < 16);
    }
  }
}

// ---------------------------------------------------------------------------
// Query tiles (prefill: many queries of one sequence share the keys).  A
// block holds 64 queries of one sequence (16 per wave, as 8 two-query A
// fragments kept in registers) and streams ST_COLS columns; every wave
// runs 8 MFMAs per 16-key fragment.
constexpr int ST_QUERIES = 64;
constexpr int ST_COLS = 512;

__global__ __launch_bounds__(256) void score_tile_kernel(ScoreArgs a, int64_t ncols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tiles_per_seq = (a.q_per_seq + ST_QUERIES - 1) / ST_QUERIES;
  const int64_t seq = blockIdx.y / tiles_per_seq;
  const int64_t qs0 = (blockIdx.y % tiles_per_seq) * ST_QUERIES + 16 * wave;   // in-sequence index
  const int64_t qend = (seq + 1) * a.q_per_seq;
  const int64_t qbase = seq * a.q_per_seq + qs0;
  const int row = lane & 15;
  i32x8 afrag[8];
  float w4[8][4];
  int64_t nvq[8];
  int64_t my_q[8];
  int64_t nv_max = 0;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    int64_t qa = qbase + 2 * f + (row >> 3);           // query of this lane's A row
    afrag[f] = load_qfrag(a.q_fp8, qa, row & 7, qa < qend, lane);
    int64_t qo = qbase + 2 * f + (lane >> 5);          // query of this lane's C rows
    my_q[f] = qo;
    bool live = qo < qend;
    int nvp = live ? visible_count(a.q_pos[qo]) : 0;
    nvq[f] = nvp < a.n_entries ? nvp : a.n_entries;
    nv_max = nvq[f] > nv_max ? nvq[f] : nv_max;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int h = 4 * ((lane >> 4) & 1) + r;
      w4[f][r] = live ? a.w[qo * IH + h] : 0.f;
    }
  }
  // wave-uniform bound on the visible columns of these 16 queries
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    int64_t o = __shfl_xor(nv_max, off);
    nv_max = o > nv_max ? o : nv_max;
  }
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  const int64_t nblk = (ncols + 7) >> 3;
  const int64_t c0 = (int64_t)blockIdx.x * ST_COLS;
  const bool owner = (lane & 16) == 0;
  for (int fc = 0; fc < ST_COLS / 16; ++fc) {
    int64_t cbase = c0 + 16 * fc;
    if (cbase >= ncols) break;
    int64_t col = cbase + (lane & 15);
    if (cbase >= nv_max) {
      // no query of this wave sees these columns
#pragma unroll
      for (int f = 0; f < 8; ++f)
        if (my_q[f] < qend)
          store_frag(-__builtin_huge_valf(), my_q[f], col, ncols, nblk, a.scores, a.block_max, lane,
                     owner);
      continue;
    }
    i32x8 b = load_kfrag(kbase, col, col < ncols && col < nv_max, lane);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_f8_16x16x128(afrag[f], b, acc);
      float s = head_sum(acc, w4[f]);
      float v = (col < nvq[f]) ? s : -__builtin_huge_valf();
      if (my_q[f] < qend)
        store_frag(v, my_q[f], col, ncols, nblk, a.scores, a.block_max, lane, owner);
    }
  }
}

int64_t score_ncols(const ScoreArgs& a) {
  return a.pool ? (int64_t)CSA_BLOCK * a.n_pool_blocks : a.n_entries;
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t st) {
  int64_t Q = a.n_seq * a.q_per_seq;
  int64_t ncols = score_ncols(a);
  if (Q == 0 || ncols == 0) return hipSuccess;
  if (a.pool) {
    dim3 grid((unsigned)((ncols + SQ_COLS - 1) / SQ_COLS), (unsigned)Q);
    hipLaunchKernelGGL(score_query_kernel<true>, grid, dim3(256), 0, st, a, ncols);
  } else if (a.q_per_seq >= 32) {
    int64_t tiles = (a.q_per_seq + ST_QUERIES - 1) / ST_QUERIES;
    dim3 grid((unsigned)((ncols + ST_COLS - 1) / ST_COLS), (unsigned)(a.n_seq * tiles));
    hipLaunchKernelGGL(score_tile_kernel, grid, dim3(256), 0, st, a, ncols);
  } else {
    dim3 grid((unsigned)((ncols + SQ_COLS - 1) / SQ_COLS), (unsigned)Q);
    hipLaunchKernelGGL(score_query_kernel<false>, grid, dim3(256), 0, st, a, ncols);
  }
  return hipGetLastError();
}

}  // namespace csa

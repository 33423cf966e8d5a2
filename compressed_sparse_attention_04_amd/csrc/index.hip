// Indexer scoring on the matrix cores.
//
// P3 §02: Full layers score every causally visible position; Reindex layers
// rescore with their own indexer query, inside the hierarchical pool.
// score_j = sum_h w_h * ReLU(q_h . k_j), 8 heads x 128 dims, E4M3 operands.
//
// The E4M3 operands are converted in registers to fp16 (exact: 4 significant
// bits, exponents 2^-9 .. 2^8) and contracted on the fp16 matrix cores with
// float32 accumulation, four v_mfma 16x16x32 per 16-row x 16-key fragment.
// Every product is exact and the sum is a float32 sum.  (The gfx950 fp8
// v_mfma 16x16x128 accumulates 128 products with about 2^-15 relative
// precision, too coarse for a Top-K that must agree with the exact scores up
// to 1e-5 near the threshold.)
//
// A fragment holds 8 heads of one query (rows 8-15 zero) or 8 heads each of
// two queries.  The epilogue applies ReLU and the head weights on the
// accumulator (lane l holds rows 4*(l/16)+r, column l%16), folds the two
// 16-lane halves that hold the 8 heads of a query, and optionally reduces 8
// adjacent columns to a block max.
#include "common.h"
#include "index_core.h"
#include "kernels.h"

namespace csa {

using namespace idxf;

// ---------------------------------------------------------------------------
// One query per block (decode, and every pooled call): the block covers
// SQ_COLS columns, each of its 4 waves SQ_COLS / 4 of them, 16 per MFMA.
// Key rows stream through whole-line loads (non-temporal for the dense scan,
// whose rows are read once) and a per-wave LDS staging slot.
constexpr int SQ_COLS = 1024;
constexpr int SQ_UNROLL = 4;

template <bool POOLED>
__global__ __launch_bounds__(256) void score_query_kernel(ScoreArgs a, int64_t ncols) {
  __shared__ uint4 stage_all[4][128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint4* stage = stage_all[wave];
  const int64_t q = blockIdx.y;
  const int64_t seq = q / a.q_per_seq;
  const int nv_pos = visible_count(a.q_pos[q]);
  const int64_t nv = nv_pos < a.n_entries ? nv_pos : a.n_entries;
  const int row = lane & 15;
  const Frag16 afrag = load_qfrag(a.q_fp8, q, row, row < IH, lane);
  float w4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int h = 4 * (lane >> 4) + r;
    w4[r] = (lane < 32) ? a.w[q * IH + h] : 0.f;
  }
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  const int64_t nblk = (ncols + 7) >> 3;
  const int64_t c_wave = (int64_t)blockIdx.x * SQ_COLS + wave * (SQ_COLS / 4);
  constexpr int NFRAG = SQ_COLS / 4 / 16;
  // pooled: lane i < 2 NFRAG holds the pool block of half i (8 columns from
  // c_wave + 8 i); every half reads it back as a wave-uniform value
  int32_t my_blk = -1;
  if (POOLED && lane < 2 * NFRAG && c_wave + 8 * lane < ncols)
    my_blk = a.pool[q * a.n_pool_blocks + ((c_wave + 8 * lane) >> 3)];
  auto half_blk = [&](int i) { return __builtin_amdgcn_readlane(my_blk, i); };
  // half h of fragment f: one whole-line load of 8 rows (lane / 8 picks the row)
  auto load_half = [&](int f, int h) {
    const int64_t col = c_wave + 16 * f + 8 * h + (lane >> 3);
    int64_t e = col;
    bool ok = col < ncols;
    if (POOLED) {
      const int32_t blk = half_blk(2 * f + h);
      ok = ok && blk >= 0;
      e = 8 * (int64_t)blk + (col & 7);
    }
    return (ok && e < nv) ? load16<!POOLED>(kbase + e * ID + 16 * stage_chunk(lane, h)) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto load_frag = [&](int f, uint4& v0, uint4& v1) {
    v0 = load_half(f, 0);
    v1 = load_half(f, 1);
  };
  // validity of the lane's output column c_wave + 16 f + lane % 16
  auto col_valid = [&](int f) {
    const int64_t col = c_wave + 16 * f + (lane & 15);
    bool ok = col < ncols;
    int64_t e = col;
    if (POOLED) {
      const int32_t b0 = half_blk(2 * f), b1 = half_blk(2 * f + 1);
      const int32_t blk = (lane & 8) ? b1 : b0;
      ok = ok && blk >= 0;
      e = 8 * (int64_t)blk + (col & 7);
    }
    return ok && e < nv;
  };
  // software pipeline: the next SQ_UNROLL fragments load while these compute
  uint4 cur[SQ_UNROLL][2], nxt[SQ_UNROLL][2];
#pragma unroll
  for (int u = 0; u < SQ_UNROLL; ++u) load_frag(u, cur[u][0], cur[u][1]);
#pragma unroll
  for (int f0 = 0; f0 < NFRAG; f0 += SQ_UNROLL) {
    if (f0 + SQ_UNROLL < NFRAG) {
#pragma unroll
      for (int u = 0; u < SQ_UNROLL; ++u) load_frag(f0 + SQ_UNROLL + u, nxt[u][0], nxt[u][1]);
    }
#pragma unroll
    for (int u = 0; u < SQ_UNROLL; ++u) {
      __builtin_amdgcn_wave_barrier();   // the previous fragment's staged reads come first
      stage[lane] = cur[u][0];
      stage[64 + lane] = cur[u][1];
      __builtin_amdgcn_wave_barrier();   // stores before the transposed reads (LDS keeps wave order)
      f32x4 acc = frag_mma(afrag, to_frag(read_staged(stage, lane)));
      float s = head_sum(acc, w4);
      int64_t col = c_wave + 16 * (f0 + u) + (lane & 15);
      float v = col_valid(f0 + u) ? s : -__builtin_huge_valf();
      store_frag(v, q, col, ncols, nblk, a.scores, POOLED ? nullptr : a.block_max, lane, lane < 16);
    }
#pragma unroll
    for (int u = 0; u < SQ_UNROLL; ++u) {
      cur[u][0] = nxt[u][0];
      cur[u][1] = nxt[u][1];
    }
  }
}

// ---------------------------------------------------------------------------
// Query tiles (prefill: many queries of one sequence share the keys).  A
// block holds 64 queries of one sequence (16 per wave, as 8 two-query A
// fragments kept in registers) and streams ST_COLS columns in rounds of two
// 16-key fragments.  Every thread loads one whole-line 16-byte chunk of the
// round after next while the waves run 8 MFMAs per fragment of the current
// round out of LDS (the staging layout of the query kernel, double-buffered,
// one barrier a round), so the four waves share one copy of the keys.
constexpr int ST_QUERIES = 64;
constexpr int ST_COLS = 512;
constexpr int ST_ROUND = 32;

// BM: also write the 8-column block maxima (a template parameter, so that the
// unrolled fragment loop has no branch and the MFMAs of one query fragment
// overlap the epilogue of another).
template <bool BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void score_tile_kernel(ScoreArgs a, int64_t ncols) {
  __shared__ uint4 stage[2][2][128];   // [buffer][fragment][slot]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qps = (int)a.q_per_seq;
  const int tiles_per_seq = (qps + ST_QUERIES - 1) / ST_QUERIES;
  const int64_t seq = blockIdx.y / tiles_per_seq;
  const int qs0 = (int)(blockIdx.y % tiles_per_seq) * ST_QUERIES + 16 * wave;   // in-sequence index
  const int64_t qseq0 = seq * a.q_per_seq;
  const int row = lane & 15;
  Frag16 afrag[8];
  float w4[8][4];
  int nvq[8];            // visible columns of the query of this lane's C rows
  uint32_t live = 0;     // bit f: that query exists
  int nv_max = 0;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int qa = qs0 + 2 * f + (row >> 3);            // query of this lane's A row
    afrag[f] = load_qfrag(a.q_fp8, qseq0 + qa, row & 7, qa < qps, lane);
    const int qo = qs0 + 2 * f + (lane >> 5);           // query of this lane's C rows
    const bool ok = qo < qps;
    live |= (uint32_t)ok << f;
    const int nvp = ok ? visible_count(a.q_pos[qseq0 + qo]) : 0;
    nvq[f] = nvp < a.n_entries ? nvp : (int)a.n_entries;
    nv_max = nvq[f] > nv_max ? nvq[f] : nv_max;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * ((lane >> 4) & 1) + r;
      w4[f][r] = ok ? a.w[(qseq0 + qo) * IH + h] : 0.f;
    }
  }
  // wave-uniform bounds on the visible columns of these 16 queries
  int nv_min = 0x7FFFFFFF;
#pragma unroll
  for (int f = 0; f < 8; ++f)
    if ((live >> f) & 1u) nv_min = nvq[f] < nv_min ? nvq[f] : nv_min;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(nv_max, off), p = __shfl_xor(nv_min, off);
    nv_max = o > nv_max ? o : nv_max;
    nv_min = p < nv_min ? p : nv_min;
  }
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  const int nblk = (int)((ncols + 7) >> 3);
  const int nc = (int)ncols;                 // < 2^23 (checked by the launcher)
  const int c0 = blockIdx.x * ST_COLS;
  // Buffer views of this tile's score / block-max rows; stores with an offset
  // past the live rows (or the OOB marker) are dropped by the hardware, which
  // replaces per-lane branches.  Row of fragment f for this lane:
  // 16 wave + 2 f + lane / 32 (the f part goes in the scalar offset).
  const int tile_q0 = (int)(blockIdx.y % tiles_per_seq) * ST_QUERIES;
  const int live_rows = (qps - tile_q0) < ST_QUERIES ? (qps - tile_q0) : ST_QUERIES;
  // scores may be absent (block maxima only): an empty view drops every store
  const bool has_sc = a.scores != nullptr;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      has_sc ? (void*)(a.scores + (qseq0 + tile_q0) * ncols) : (void*)a.block_max, (short)0,
      has_sc ? live_rows * nc * 4 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t brs = BM ?
      __builtin_amdgcn_make_buffer_rsrc(a.block_max + (qseq0 + tile_q0) * (int64_t)nblk, (short)0, live_rows * nblk * 4,
                                        0x00020000) : srs;
  constexpr uint32_t OOB = 0x80000000u;
  const int lrow = 16 * wave + (lane >> 5);
  // this thread's chunk of every round: fragment fr, half h, staging slot 64 h + li
  const int fr = tid >> 7, h = (tid >> 6) & 1, li = tid & 63;
  const int n_row = 8 * h + (li >> 3);
  const int chunk = stage_chunk(li, h);
  auto load_round = [&](int r) {
    const int col = c0 + ST_ROUND * r + 16 * fr + n_row;
    return col < nc ? *reinterpret_cast<const uint4*>(kbase + (int64_t)col * ID + 16 * chunk)
                    : make_uint4(0u, 0u, 0u, 0u);
  };
  constexpr int N_ROUNDS = ST_COLS / ST_ROUND;
  stage[0][fr][64 * h + li] = load_round(0);
  uint4 nxt = load_round(1);
  for (int r = 0; r < N_ROUNDS; ++r) {
    __syncthreads();   // round r is in buffer r & 1; the other buffer's readers are done
    if (r + 1 < N_ROUNDS) stage[(r + 1) & 1][fr][64 * h + li] = nxt;
    if (r + 2 < N_ROUNDS) nxt = load_round(r + 2);
#pragma unroll 1
    for (int f2 = 0; f2 < 2; ++f2) {
      const int cbase = c0 + ST_ROUND * r + 16 * f2;
      if (cbase >= nc) break;
      const int col = cbase + (lane & 15);
      const uint32_t vo_s = (has_sc && col < nc && (lane & 16) == 0) ? (uint32_t)(lrow * nc + col) * 4u : OOB;
      const uint32_t vo_b = (BM && col < nc && (lane & 23) == 0) ? (uint32_t)(lrow * nblk + (col >> 3)) * 4u : OOB;
      if (cbase >= nv_max) {
        // no query of this wave sees these columns
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-__builtin_huge_valf()), srs, vo_s, 2 * f * nc * 4, 0);
          if (BM) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-__builtin_huge_valf()), brs, vo_b, 2 * f * nblk * 4, 0);
        }
        continue;
      }
      const bool all_visible = cbase + 16 <= nv_min;
      const Frag16 b = to_frag(read_staged(stage[r & 1][f2], lane));
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const f32x4 acc = frag_mma(afrag[f], b);
        float v = head_sum(acc, w4[f]);
        if (!all_visible) v = (col < nvq[f]) ? v : -__builtin_huge_valf();
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), srs, vo_s, 2 * f * nc * 4, 0);
        if (BM) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score_max8(v)), brs, vo_b, 2 * f * nblk * 4, 0);
      }
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
  } else if (a.q_per_seq >= 32 && ncols < (int64_t(1) << 23)) {   // 32-bit buffer offsets
    int64_t tiles = (a.q_per_seq + ST_QUERIES - 1) / ST_QUERIES;
    dim3 grid((unsigned)((ncols + ST_COLS - 1) / ST_COLS), (unsigned)(a.n_seq * tiles));
    if (a.block_max) hipLaunchKernelGGL(score_tile_kernel<true>, grid, dim3(256), 0, st, a, ncols);
    else hipLaunchKernelGGL(score_tile_kernel<false>, grid, dim3(256), 0, st, a, ncols);
  } else {
    dim3 grid((unsigned)((ncols + SQ_COLS - 1) / SQ_COLS), (unsigned)Q);
    hipLaunchKernelGGL(score_query_kernel<false>, grid, dim3(256), 0, st, a, ncols);
  }
  return hipGetLastError();
}

}  // namespace csa

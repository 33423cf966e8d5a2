// Indexer scoring on the matrix cores.
//
// "DeepSeek-V4.1 架构解析" §02: Full layers score every causally visible position; Reindex layers
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
// Pooled scoring, one query per block: the block covers SQ_COLS pooled
// columns, each of its 4 waves SQ_COLS / 4 of them, 16 per MFMA.  Key rows
// (1 KiB pool blocks) stream through whole-line loads and a per-wave LDS
// staging slot, in groups of SQ_UNROLL fragments held in two register sets
// used in turn (the next group loads while this one computes, and no
// register with a load in flight is copied).  Loads are unconditional: a
// column outside the pool's visible entries reads entry 0 and scores -inf.
// Stores go through a buffer view of the query's row (out-of-range offsets
// are dropped), so no branch surrounds a memory operation.
constexpr int SQ_COLS = 1024;
constexpr int SQ_UNROLL = 4;

__global__ __launch_bounds__(256) void score_pool_kernel(ScoreArgs a, int64_t ncols) {
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
  const int64_t c_wave = (int64_t)blockIdx.x * SQ_COLS + wave * (SQ_COLS / 4);
  constexpr int NFRAG = SQ_COLS / 4 / 16;
  constexpr int NGRP = NFRAG / SQ_UNROLL;
  // lane i < 2 NFRAG holds the pool block of half i (8 columns from
  // c_wave + 8 i); every half reads it back as a wave-uniform value
  int32_t my_blk = -1;
  if (lane < 2 * NFRAG && c_wave + 8 * lane < ncols)
    my_blk = a.pool[q * a.n_pool_blocks + ((c_wave + 8 * lane) >> 3)];
  // Half i = one pool block of 8 columns.  Lane i keeps the number of its
  // visible entries (cnt) and its block; every half reads them back as
  // wave-uniform values.  32-bit: entries < 2^30.
  // (a block id outside the visible entries, or a bogus one from the caller,
  // has no visible entry; the test comes before the multiply, so 8 * id
  // stays below 2^30)
  const int nv_i = (int)nv;
  const bool in_range = my_blk >= 0 && my_blk <= (nv_i >> 3);
  const int rem = in_range ? nv_i - 8 * my_blk : 0;
  const int my_cnt = rem <= 0 ? 0 : (rem >= 8 ? 8 : rem);
  const int my_blkc = my_cnt > 0 ? my_blk : 0;
  // one word per half (block id < 2^27 above the count), one readlane each
  const int my_pack = (my_blkc << 4) | my_cnt;
  auto half_cnt = [&](int i) { return __builtin_amdgcn_readlane(my_pack, i) & 15; };
  // a buffer view of half i's visible rows (built on the scalar unit): rows
  // at or past the count read past the view and get zeros, so the lane's
  // offset needs no per-half selection and no 64-bit address
  auto half_view = [&](int i) {
    const int pk = __builtin_amdgcn_readlane(my_pack, i);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)(pk >> 4) * (8 * ID)), (short)0,
                                             (pk & 15) * ID, 0x00020000);
  };
  // lane's byte offsets inside a half: row lane / 8, whole-line chunk of half h
  const int lrow_k = lane >> 3;
  const uint32_t off_row[2] = {(uint32_t)(lrow_k * ID + 16 * stage_chunk(lane, 0)),
                               (uint32_t)(lrow_k * ID + 16 * stage_chunk(lane, 1))};
  // half h of fragment f: one whole-line load of 8 rows (lane / 8 picks the row)
  auto load_group = [&](int grp, uint4 (&v)[SQ_UNROLL][2]) {
#pragma unroll
    for (int u = 0; u < SQ_UNROLL; ++u) {
      const int f = grp * SQ_UNROLL + u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(half_view(2 * f + h), off_row[h], 0, 0);
        v[u][h] = make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
      }
    }
  };
  constexpr uint32_t OOB = 0x80000000u;
  // (pooled mode always has a score array; an absent one gets an empty view)
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      a.scores ? (void*)(a.scores + q * ncols) : (void*)a.k_fp8, (short)0, a.scores ? (int)(ncols * 4) : 0,
      0x00020000);
  const int ncols_i = (int)ncols;                     // <= 8 x 65,536
  const int cw = (int)c_wave;
  // The group's four fragments (64 consecutive columns) go out as one store
  // with every lane: fragment u's scores sit in lanes 0-31 after the head
  // sums, rows 0 and 1 take fragments 0 and 1 and one v_permlane32_swap
  // brings fragments 2 and 3 into rows 2 and 3, so lane l holds column l.
  static_assert(SQ_UNROLL == 4, "one store per group of four fragments");
  const uint32_t vo0 = (uint32_t)(cw + lane) * 4u;
  auto compute_group = [&](int grp, const uint4 (&v)[SQ_UNROLL][2]) {
    float sc[SQ_UNROLL];
    uint64_t valid = 0;
#pragma unroll
    for (int u = 0; u < SQ_UNROLL; ++u) {
      const int f = grp * SQ_UNROLL + u;
      __builtin_amdgcn_wave_barrier();   // the previous fragment's staged reads come first
      stage[lane] = v[u][0];
      stage[64 + lane] = v[u][1];
      __builtin_amdgcn_wave_barrier();   // stores before the transposed reads (LDS keeps wave order)
      sc[u] = head_sum(frag_mma(afrag, to_frag(read_staged(stage, lane))), w4);
      // column c of fragment u is valid when its offset in its pool block
      // (c % 8) is below that block's visible count: bits 16 u .. of a
      // wave-uniform mask built from the halves' counts (<= 8) on the scalar unit
      const uint32_t m16 = ((1u << half_cnt(2 * f)) - 1u) | (((1u << half_cnt(2 * f + 1)) - 1u) << 8);
      valid |= (uint64_t)m16 << (16 * u);
    }
    const bool odd_row = (lane & 16) != 0;
    const float v01 = odd_row ? sc[1] : sc[0], v23 = odd_row ? sc[3] : sc[2];
    const float s64 = __uint_as_float(
        __builtin_amdgcn_permlane32_swap(__float_as_uint(v01), __float_as_uint(v23), false, false)[0]);
    const float v_out = __builtin_amdgcn_inverse_ballot_w64(valid) ? s64 : -__builtin_huge_valf();
    // a column at or past ncols is past the view's records and its store is
    // dropped (the range check covers the immediate offset, where 256 grp goes)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v_out), srs, vo0 + 256u * (uint32_t)grp, 0, 0);
  };
  if (nv == 0) {
    // nothing visible: every column is -inf, and no key row may be read (the
    // key array can be empty)
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      const int col = cw + 16 * f + (lane & 15);
      const uint32_t vo = (lane < 16 && col < ncols_i) ? (uint32_t)col * 4u : OOB;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-__builtin_huge_valf()), srs, vo, 0, 0);
    }
    return;
  }
  uint4 ra[SQ_UNROLL][2], rb[SQ_UNROLL][2];
  load_group(0, ra);
#pragma unroll
  for (int grp = 0; grp < NGRP; grp += 2) {
    if (grp + 1 < NGRP) load_group(grp + 1, rb);
    compute_group(grp, ra);
    if (grp + 2 < NGRP) load_group(grp + 2, ra);
    if (grp + 1 < NGRP) compute_group(grp + 1, rb);
  }
}

// ---------------------------------------------------------------------------
// Dense scan of one query per block row, persistent over column chunks: block
// (b, q) takes the SQ_COLS-column chunks b, b + gridDim.x, ... of query q, so
// the query fragment, the weights and the visible count are loaded once per
// block, and each wave runs one software pipeline over all its fragments
// (256 columns per chunk, SC_GROUP fragments per group, two register sets
// used in turn so that no register with a load in flight is copied).  Key
// loads are unconditional: a column past the visible entries reads entry 0
// and its score is replaced by -inf (an MFMA column only reaches its own
// output column), so the compiler can count the loads in flight instead of
// waiting for all of them.
constexpr int SC_BLOCKS = 2048;   // ~four rounds of two 4-wave blocks per CU (240 registers); 512 and 4,096 measured slower

// SC_GROUP: 8 fragments when a block streams several chunks (4 measured 2%
// slower there: fewer bytes in flight per wave), 4 when it has one chunk
// (two groups of 8 would leave nothing to overlap).  COLS: the chunk; a scan
// too small to give 256 blocks of 1,024 columns (one short sequence) takes
// chunks of 256 columns instead, one group per wave, so its blocks do not
// run four groups one after another.
template <int SC_GROUP, int COLS = SQ_COLS>
__global__ __launch_bounds__(256) void score_scan_kernel(ScoreArgs a, int64_t ncols) {
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
  for (int r = 0; r < 4; ++r) w4[r] = (lane < 32) ? a.w[q * IH + 4 * (lane >> 4) + r] : 0.f;
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  const int64_t nblk = (ncols + 7) >> 3;
  constexpr int NFRAG = COLS / 4 / 16;   // fragments of a wave per chunk
  // outputs through buffer stores: no branch around a store, so the compiler
  // can count the memory operations in flight (stores count with the loads)
  constexpr uint32_t OOB = 0x80000000u;
  float* const any_out = a.scores ? a.scores : a.block_max;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      a.scores ? (void*)(a.scores + q * ncols) : (void*)any_out, (short)0, a.scores ? (int)(ncols * 4) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      a.block_max ? (void*)(a.block_max + q * nblk) : (void*)any_out, (short)0, a.block_max ? (int)(nblk * 4) : 0,
      0x00020000);
  const int64_t n_chunks = (ncols + COLS - 1) / COLS;
  const int64_t my_chunks = blockIdx.x < n_chunks ? (n_chunks - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int n_groups = (int)(my_chunks * (NFRAG / SC_GROUP));
  // first column of fragment g of this wave's stream.  With 8-fragment
  // groups (several chunks per block) each wave reads its own quarter of the
  // chunk; with 4-fragment groups (one chunk per block) the four waves take
  // the chunk's 64-column groups in turn, so the block's loads in flight sit
  // side by side (1-2 % faster there, ~1 % slower with 8-fragment groups).
  auto frag_col = [&](int g) {
    const int64_t chunk = blockIdx.x + (int64_t)gridDim.x * (g / NFRAG);
    const int gi = g % NFRAG;
    if constexpr (SC_GROUP == 4)
      return chunk * COLS + ((gi / SC_GROUP) * 4 + wave) * (SC_GROUP * 16) + 16 * (gi % SC_GROUP);
    else
      return chunk * COLS + wave * (COLS / 4) + 16 * gi;
  };
  auto load_group = [&](int grp, uint4 (&v)[SC_GROUP][2]) {
#pragma unroll
    for (int u = 0; u < SC_GROUP; ++u) {
      const int64_t c0 = frag_col(grp * SC_GROUP + u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t col = c0 + 8 * h + (lane >> 3);
        const int64_t e = (grp < n_groups && col < ncols && col < nv) ? col : 0;
        v[u][h] = load16<true>(kbase + e * ID + 16 * stage_chunk(lane, h));
      }
    }
  };
  // Four consecutive fragments (64 consecutive columns) go out together: the
  // head sums leave fragment u's scores in lanes 0-31 (16-lane rows 0 and 1
  // alike), so rows 0 and 1 take fragments u, u + 1 and one
  // v_permlane32_swap brings fragments u + 2, u + 3 into rows 2 and 3; lane l
  // then holds column l of the 64, and one store instruction with every lane
  // (and one block-max step over the 64) replaces four with 16 lanes each.
  // Fewer store instructions leave more of the memory counter to the key
  // loads in flight.
  static_assert(SC_GROUP % 4 == 0 && NFRAG % 4 == 0, "fragments go out in fours within a chunk");
  auto compute_group = [&](int grp, const uint4 (&v)[SC_GROUP][2]) {
    const bool odd_row = (lane & 16) != 0;
#pragma unroll
    for (int u0 = 0; u0 < SC_GROUP; u0 += 4) {
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_wave_barrier();   // the previous fragment's staged reads come first
        stage[lane] = v[u0 + i][0];
        stage[64 + lane] = v[u0 + i][1];
        __builtin_amdgcn_wave_barrier();   // stores before the transposed reads (LDS keeps wave order)
        sc[i] = head_sum(frag_mma(afrag, to_frag(read_staged(stage, lane))), w4);
      }
      const float v01 = odd_row ? sc[1] : sc[0], v23 = odd_row ? sc[3] : sc[2];
      const float s64 = __uint_as_float(
          __builtin_amdgcn_permlane32_swap(__float_as_uint(v01), __float_as_uint(v23), false, false)[0]);
      const int64_t col = frag_col(grp * SC_GROUP + u0) + lane;
      const float v_out = (col < ncols && col < nv) ? s64 : -__builtin_huge_valf();
      const float m_out = score_max8(v_out);
      // lanes 0, 8, .. own the block maxima; a missing output stores out of
      // range, which is dropped
      const uint32_t vo_s = col < ncols ? (uint32_t)col * 4u : OOB;
      const uint32_t vo_b = ((lane & 7) == 0 && (col >> 3) < nblk) ? (uint32_t)(col >> 3) * 4u : OOB;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v_out), srs, vo_s, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_out), brs, vo_b, 0, 0);
    }
  };
  uint4 ra[SC_GROUP][2], rb[SC_GROUP][2];
  if (n_groups > 0) load_group(0, ra);
  int grp = 0;
  for (; grp + 1 < n_groups; grp += 2) {
    load_group(grp + 1, rb);
    compute_group(grp, ra);
    if (grp + 2 < n_groups) load_group(grp + 2, ra);
    compute_group(grp + 1, rb);
  }
  if (grp < n_groups) compute_group(grp, ra);
}

// ---------------------------------------------------------------------------
// Query tiles (prefill: many queries of one sequence share the keys).  A
// block holds 64 queries of one sequence (16 per wave, as 8 two-query A
// fragments kept in registers) and streams ST_COLS columns in rounds of four
// 16-key fragments.  Every thread loads two whole-line 16-byte chunks of the
// round after next while the waves run 8 MFMAs per k-step of each fragment of
// the current round out of LDS (the staging layout of the query kernel,
// double-buffered, one barrier a round), so the four waves share one copy of
// the keys.  A fragment's epilogue overlaps the next fragment's MFMAs.  (With
// 8 independent accumulator chains per wave the matrix pipe sustains about
// 1.19 PFLOP/s on this instruction, 16 chains about 1.7; 16 chains, as two
// key fragments x 8 query pairs or four x 4, did not fit the epilogue's
// overlap and the 256 registers of two waves per SIMD and ran slower.)
constexpr int ST_QUERIES = 64;
constexpr int ST_COLS = 512;
constexpr int ST_ROUND = 64;
constexpr int ST_FR = ST_ROUND / 16;   // key fragments per round

// BM: also write the 8-column block maxima (a template parameter, so that the
// unrolled fragment loop has no branch and the MFMAs of one query fragment
// overlap the epilogue of another).
template <bool BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void score_tile_kernel(ScoreArgs a, int64_t ncols) {
  __shared__ uint4 stage[2][ST_FR][128];   // [buffer][fragment][slot]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qps = (int)a.q_per_seq;
  const int tiles_per_seq = (qps + ST_QUERIES - 1) / ST_QUERIES;
  const int64_t seq = blockIdx.y / tiles_per_seq;
  const int qs0 = (int)(blockIdx.y % tiles_per_seq) * ST_QUERIES + 16 * wave;   // in-sequence index
  const int64_t qseq0 = seq * a.q_per_seq;
  const int row = lane & 15;
  // After the paired head sums (head_sum_pair over query pairs 2p and 2p+1),
  // lane l holds the score of wave query 4p + vrow, vrow = 2 ((l / 16) & 1) + l / 32.
  const int vrow = 2 * ((lane >> 4) & 1) + (lane >> 5);
  Frag16 afrag[8];
  float w4[8][4];
  int nvs[4];            // visible columns of this lane's output query, per pair set
  int nv_min = 0x7FFFFFFF;
  {
    // every load first, from clamped (existing) queries, then the conversions:
    // a load under a branch, or a use right after it, would cost one round
    // trip per query pair
    Raw32 rq[8];
    int32_t pq[4];
    float wq[8][4];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int qa = qs0 + 2 * f + (row >> 3);          // query of this lane's A row
      const int qo = qs0 + 2 * f + (lane >> 5);         // query of this lane's C rows
      const int64_t qac = qseq0 + (qa < qps ? qa : qps - 1), qoc = qseq0 + (qo < qps ? qo : qps - 1);
      rq[f] = load_raw32(a.q_fp8 + (qac * IH + (row & 7)) * ID, true, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) wq[f][r] = a.w[qoc * IH + 4 * ((lane >> 4) & 1) + r];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qv = qs0 + 4 * p + vrow;
      pq[p] = a.q_pos[qseq0 + (qv < qps ? qv : qps - 1)];
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int qa = qs0 + 2 * f + (row >> 3);
      const int qo = qs0 + 2 * f + (lane >> 5);
      const Raw32 z = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
      afrag[f] = to_frag(qa < qps ? rq[f] : z);
#pragma unroll
      for (int r = 0; r < 4; ++r) w4[f][r] = qo < qps ? wq[f][r] : 0.f;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool ok = qs0 + 4 * p + vrow < qps;
      const int nvp = ok ? visible_count(pq[p]) : 0;
      nvs[p] = nvp < a.n_entries ? nvp : (int)a.n_entries;
      if (ok) nv_min = nvs[p] < nv_min ? nvs[p] : nv_min;
    }
  }
  // wave-uniform bound on the visible columns of these 16 queries (scalar,
  // so the masking below is a branch, taken only on partly visible fragments)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(nv_min, off);
    nv_min = o < nv_min ? o : nv_min;
  }
  nv_min = __builtin_amdgcn_readfirstlane(nv_min);
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  const int nblk = (int)((ncols + 7) >> 3);
  const int nc = (int)ncols;                 // < 2^23 (checked by the launcher)
  const int c0 = blockIdx.x * ST_COLS;
  // Buffer views of this tile's score / block-max rows, one per pair set p
  // (rows 4p .. of the tile, holding only the live rows from there on), so the
  // hardware's bounds check drops the stores of absent queries and of the
  // out-of-range marker; the offset is the lane's voffset alone.
  const int tile_q0 = (int)(blockIdx.y % tiles_per_seq) * ST_QUERIES;
  const int live_rows = (qps - tile_q0) < ST_QUERIES ? (qps - tile_q0) : ST_QUERIES;
  const bool has_sc = a.scores != nullptr;
  __amdgpu_buffer_rsrc_t srs[4], brs[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int rows = live_rows - 4 * p > 0 ? live_rows - 4 * p : 0;
    srs[p] = __builtin_amdgcn_make_buffer_rsrc(
        has_sc ? (void*)(a.scores + (qseq0 + tile_q0 + 4 * p) * ncols) : (void*)a.k_fp8, (short)0,
        has_sc ? rows * nc * 4 : 0, 0x00020000);
    brs[p] = BM ? __builtin_amdgcn_make_buffer_rsrc(a.block_max + (qseq0 + tile_q0 + 4 * p) * (int64_t)nblk,
                                                    (short)0, rows * nblk * 4, 0x00020000)
                : srs[p];
  }
  constexpr uint32_t OOB = 0x80000000u;
  const int lrow = 16 * wave + vrow;
  // this thread's chunks of every round: fragment 2 sub + fr (sub = 0, 1),
  // half h, staging slot 64 h + li
  const int fr = tid >> 7, h = (tid >> 6) & 1, li = tid & 63;
  const int n_row = 8 * h + (li >> 3);
  const int chunk = stage_chunk(li, h);
  constexpr int N_ROUNDS = ST_COLS / ST_ROUND;
  static_assert(N_ROUNDS % 2 == 0, "rounds go in pairs (two register sets)");
  // Key bytes through a view of the sequence's first nc rows: a column at or
  // past nc, or a round past the block's last, reads past the view and gets
  // zeros.  The loads are unconditional, so the compiler counts the memory
  // operations in flight: a round waits only for the key loads issued a
  // round earlier, never for the score stores issued since.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nc * ID, 0x00020000);
  auto load_round = [&](int r, int sub) {
    const int col = c0 + ST_ROUND * r + 32 * sub + 16 * fr + n_row;
    const uint32_t off = (r < N_ROUNDS && col < nc) ? (uint32_t)col * ID + 16u * (uint32_t)chunk : OOB;
    const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
    return make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
  };
  // Round r: the keys of round r + 1 (held) go to the other staging buffer
  // after the loads of round r + 2 (into spare) are issued, then the round's
  // fragments are computed from buffer r & 1.
  auto round = [&](int r, uint4 (&held)[2], uint4 (&spare)[2]) {
    __syncthreads();   // round r is in buffer r & 1; the other buffer's readers are done
    spare[0] = load_round(r + 2, 0);
    spare[1] = load_round(r + 2, 1);
    stage[(r + 1) & 1][fr][64 * h + li] = held[0];
    stage[(r + 1) & 1][2 + fr][64 * h + li] = held[1];
    // Each key fragment against the wave's 8 query pairs: 8 independent
    // accumulators with the k-steps interleaved across them (a chain of
    // dependent MFMAs on one accumulator would wait on each result), then
    // the epilogues, two query pairs per cross-lane swap.
    const int rbase = c0 + ST_ROUND * r;
    if (rbase >= nc) return;   // uniform: nothing of this round is a column
#pragma unroll
    for (int f2 = 0; f2 < ST_FR; ++f2) {
      const int cbase = rbase + 16 * f2;
      const Frag16 b = to_frag(read_staged(stage[r & 1][f2], lane));
      f32x4 acc[8];
#pragma unroll
      for (int f = 0; f < 8; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int f = 0; f < 8; ++f) acc[f] = mfma_f16_16x16x32(afrag[f].s[ks], b.s[ks], acc[f]);
      const int col = cbase + (lane & 15);
      const uint32_t vo_s = col < nc ? (uint32_t)(lrow * nc + col) * 4u : OOB;
      const uint32_t vo_b = (col < nc && (lane & 7) == 0) ? (uint32_t)(lrow * nblk + (col >> 3)) * 4u : OOB;
      float v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) v[p] = head_sum_pair(acc[2 * p], w4[2 * p], acc[2 * p + 1], w4[2 * p + 1]);
      // columns a query does not see (or past the row) score -inf
      if (cbase + 16 > nv_min) {
#pragma unroll
        for (int p = 0; p < 4; ++p) v[p] = col < nvs[p] ? v[p] : -__builtin_huge_valf();
      }
      if (has_sc) {
#pragma unroll
        for (int p = 0; p < 4; ++p) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[p]), srs[p], vo_s, 0, 0);
      }
      if (BM) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score_max8(v[p])), brs[p], vo_b, 0, 0);
      }
    }
  };
  uint4 ra[2], rb[2];
  stage[0][fr][64 * h + li] = load_round(0, 0);
  stage[0][2 + fr][64 * h + li] = load_round(0, 1);
  ra[0] = load_round(1, 0);
  ra[1] = load_round(1, 1);
  for (int r = 0; r < N_ROUNDS; r += 2) {
    round(r, ra, rb);
    round(r + 1, rb, ra);
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
    hipLaunchKernelGGL(score_pool_kernel, grid, dim3(256), 0, st, a, ncols);
  } else if (a.q_per_seq >= 32 && ncols < (int64_t(1) << 23)) {   // 32-bit buffer offsets
    int64_t tiles = (a.q_per_seq + ST_QUERIES - 1) / ST_QUERIES;
    dim3 grid((unsigned)((ncols + ST_COLS - 1) / ST_COLS), (unsigned)(a.n_seq * tiles));
    if (a.block_max) hipLaunchKernelGGL(score_tile_kernel<true>, grid, dim3(256), 0, st, a, ncols);
    else hipLaunchKernelGGL(score_tile_kernel<false>, grid, dim3(256), 0, st, a, ncols);
  } else {
    // about SC_BLOCKS blocks, every block of a query with the same number of chunks
    const int64_t n_chunks = (ncols + SQ_COLS - 1) / SQ_COLS;
    int64_t per_q = (SC_BLOCKS + Q - 1) / Q;
    per_q = per_q < n_chunks ? per_q : n_chunks;
    const int64_t chunks_per_block = (n_chunks + per_q - 1) / per_q;
    per_q = (n_chunks + chunks_per_block - 1) / chunks_per_block;
    dim3 grid((unsigned)per_q, (unsigned)Q);
    if (ncols >= ((int64_t)1 << 29)) return hipErrorInvalidValue;   // 32-bit buffer offsets
    if (Q * n_chunks < 256) {
      constexpr int SMALL = 256;
      const dim3 g2((unsigned)((ncols + SMALL - 1) / SMALL), (unsigned)Q);
      hipLaunchKernelGGL((score_scan_kernel<4, SMALL>), g2, dim3(256), 0, st, a, ncols);
    } else if (chunks_per_block >= 2) {
      hipLaunchKernelGGL(score_scan_kernel<8>, grid, dim3(256), 0, st, a, ncols);
    } else {
      hipLaunchKernelGGL(score_scan_kernel<4>, grid, dim3(256), 0, st, a, ncols);
    }
  }
  return hipGetLastError();
}

}  // namespace csa

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
#include "kernels.h"

namespace csa {

namespace {

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

// Weighted ReLU head sum of one accumulator fragment; lanes 0-15 end with the
// score of the first query (rows 0-7), lanes 32-47 with the second (rows 8-15).
// The head weights are >= 0, so every score is >= +0 (or -inf where masked).
__device__ __forceinline__ float head_sum(f32x4 acc, const float w4[4]) {
  float s = w4[0] * relu(acc[0]);
  s = fmaf(w4[1], relu(acc[1]), s);
  s = fmaf(w4[2], relu(acc[2]), s);
  s = fmaf(w4[3], relu(acc[3]), s);
  return sum_xor16(s);
}

// Max over aligned groups of 8 lanes for scores (>= +0 or -inf): on that
// set the float order is the int32 order of the bit patterns, so the DPP
// steps are integer maxes.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false); }
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

}  // namespace

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
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(a.scores + (qseq0 + tile_q0) * ncols, (short)0, live_rows * nc * 4, 0x00020000);
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
      const uint32_t vo_s = (col < nc && (lane & 16) == 0) ? (uint32_t)(lrow * nc + col) * 4u : OOB;
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

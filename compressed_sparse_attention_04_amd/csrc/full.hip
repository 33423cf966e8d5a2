// Fused Full-layer selection: the block pool, then the Top-K by rescoring
// only the entries of the best blocks.
//
// P3 §02: a Full layer scores every causally visible entry, keeps the
// Top-512, and (hierarchical pool) the 2,048 blocks of 8 entries with the
// largest block max.  Every Top-K entry lies in one of the top_k blocks by
// block max (equal maxima go to the lower block, the same rule as for
// entries): a block ranked above a block that holds a Top-K entry e has a max
// >= s(e), with equality only for a lower block, whose tying entry precedes e
// and is therefore in the Top-K as well.  So the dense scan writes only the
// block maxima, and this kernel rescores the 8 top_k entries of those blocks
// with the scan's own arithmetic (the same fragments and fp32 sums, so the
// same bits) and selects among them.
//
// One 1024-thread block per query:
//   A. pool = the NB best blocks (ascending ids, -1 padded); when the pool is
//      larger than top_k, the top_k best blocks are selected from the pool's
//      own block maxima;
//   B. each wave rescores 16 entries (two blocks) at a time: whole-line key
//      loads (four fragments ahead) staged through LDS, one 16 x 16 x 32 MFMA
//      fragment per query;
//   C. the Top-K of the rescored entries (ascending ids, -1 padded).
#include "common.h"
#include "index_core.h"
#include "kernels.h"
#include "select_core.h"

namespace csa {

using namespace sel;
using namespace idxf;

constexpr int FS_THREADS = 1024;
constexpr int FS_WAVES = FS_THREADS / 64;
constexpr int FS_KMAX = 1024;     // top_k handled here (8 top_k entries are rescored)

struct FullSelArgs {
  const float* block_max;   // [Q, nblk]
  int64_t nblk;
  int32_t NB;               // pool blocks (== K without a pool)
  int32_t* pool_out;        // [Q, NB] or null
  int32_t K;                // top_k <= FS_KMAX
  int32_t* idx;             // [Q, K]
  const uint8_t* q_fp8;     // [Q, 8, 128]
  const float* w;           // [Q, 8]
  const int32_t* q_pos;     // [Q]
  int64_t q_per_seq;
  const uint8_t* k_fp8;     // [n_seq, k_rows, 128]
  int64_t k_rows, n_entries;
};

template <int PER, int PER2>   // block maxima per thread; rescored entries per thread
__global__ __launch_bounds__(FS_THREADS) void full_select_kernel(FullSelArgs a) {
  __shared__ SelShared s;
  __shared__ int32_t pool[SEL_POOL_MAX];
  __shared__ int32_t top[FS_KMAX];
  __shared__ float sc[8 * FS_KMAX];
  __shared__ uint4 stage_all[FS_WAVES][128];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.y;
  const int NB = a.NB, K = a.K;

  // ---- A. pool, and the top_k blocks ------------------------------------------
  {
    const int pw = 64 * PER * wv + lane;
    const float* row = a.block_max + q * a.nblk;
    {
      uint32_t key[PER];
      load_keys<PER>(row, pw, (int)a.nblk, key);
      const uint32_t n_pool = block_select<FS_THREADS, PER>(s, key, (uint32_t)NB, [&](int p, uint32_t, uint32_t slot) {
        pool[slot] = p;
        if (a.pool_out) a.pool_out[q * NB + slot] = p;
      });
      for (int j = (int)n_pool + tid; j < NB; j += FS_THREADS) {
        pool[j] = -1;
        if (a.pool_out) a.pool_out[q * NB + j] = -1;
      }
    }
    if (NB > K) {
      // the top_k blocks are among the pool: select them from the pool's own
      // block maxima (pool order is id order, so ties still go to lower ids)
      __syncthreads();   // pool is complete
      constexpr int PP = SEL_POOL_MAX / FS_THREADS;
      const int pp = 64 * PP * wv + lane;
      uint32_t key[PP];
      {
        int32_t b[PP];
        float v[PP];
#pragma unroll
        for (int u = 0; u < PP; ++u) {
          const int i = pp + 64 * u;
          b[u] = i < NB ? pool[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < PP; ++u) v[u] = row[b[u] >= 0 ? b[u] : 0];   // unconditional: loads overlap
#pragma unroll
        for (int u = 0; u < PP; ++u) key[u] = b[u] >= 0 ? select_key(v[u]) : 0u;
      }
      const uint32_t n_top = block_select<FS_THREADS, PP>(s, key, (uint32_t)K, [&](int i, uint32_t, uint32_t slot) {
        top[slot] = pool[i];
      });
      for (int j = (int)n_top + tid; j < K; j += FS_THREADS) top[j] = -1;
    } else {
      __syncthreads();   // pool is complete
      for (int j = tid; j < K; j += FS_THREADS) top[j] = pool[j];
    }
  }
  __syncthreads();

  // ---- B. rescore the entries of the top_k blocks ---------------------------
  {
    const int64_t seq = q / a.q_per_seq;
    const int nv_pos = visible_count(a.q_pos[q]);
    const int64_t nv = nv_pos < a.n_entries ? nv_pos : a.n_entries;
    const int rowa = lane & 15;
    const Frag16 afrag = load_qfrag(a.q_fp8, q, rowa, rowa < IH, lane);
    float w4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w4[r] = (lane < 32) ? a.w[q * IH + 4 * (lane >> 4) + r] : 0.f;
    const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
    uint4* stage = stage_all[wv];
    const int n_frag = (K + 1) / 2;   // two blocks per 16-entry fragment; wave wv takes f = wv + 16 i
    if (nv == 0) {   // nothing visible: every rescored slot is empty (and no row may be read)
      for (int i = tid; i < 16 * n_frag; i += FS_THREADS) sc[i] = -__builtin_huge_valf();
    } else {
      // unconditional loads, an empty slot reading entry 0 (nv >= 1 here): its
      // score is replaced by -inf below, and a column of an MFMA fragment
      // affects only its own output column, so its bytes do not matter
      auto load_frag = [&](int f, uint4& v0, uint4& v1) {
        uint4 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int bi = 2 * f + h;
          const int32_t blk = (f < n_frag && bi < K) ? top[bi] : -1;
          const int64_t e = 8 * (int64_t)blk + (lane >> 3);
          v[h] = load16<false>(kbase + ((blk >= 0 && e < nv) ? e : 0) * ID + 16 * stage_chunk(lane, h));
        }
        v0 = v[0];
        v1 = v[1];
      };
      // groups of FS_GROUP fragments per wave, the next group's loads in flight
      constexpr int FS_GROUP = 4;
      const int n_mine = (n_frag - wv + FS_WAVES - 1) / FS_WAVES;
      uint4 cur[FS_GROUP][2], nxt[FS_GROUP][2];
#pragma unroll
      for (int u = 0; u < FS_GROUP; ++u) load_frag(wv + FS_WAVES * u, cur[u][0], cur[u][1]);
      for (int g0 = 0; g0 < n_mine; g0 += FS_GROUP) {
        if (g0 + FS_GROUP < n_mine) {
#pragma unroll
          for (int u = 0; u < FS_GROUP; ++u)
            load_frag(wv + FS_WAVES * (g0 + FS_GROUP + u), nxt[u][0], nxt[u][1]);
        }
#pragma unroll
        for (int u = 0; u < FS_GROUP; ++u) {
          const int f = wv + FS_WAVES * (g0 + u);
          if (g0 + u >= n_mine) break;
          __builtin_amdgcn_wave_barrier();
          stage[lane] = cur[u][0];
          stage[64 + lane] = cur[u][1];
          __builtin_amdgcn_wave_barrier();
          const f32x4 acc = frag_mma(afrag, to_frag(read_staged(stage, lane)));
          const float sco = head_sum(acc, w4);
          // lane n < 16 holds column n: entry 8 top[2 f + n / 8] + n % 8
          const int bi = 2 * f + ((lane & 15) >> 3);
          const int32_t blk = bi < K ? top[bi] : -1;
          const int64_t e = 8 * (int64_t)blk + (lane & 7);
          if (lane < 16) sc[16 * f + lane] = (blk >= 0 && e < nv) ? sco : -__builtin_huge_valf();
        }
#pragma unroll
        for (int u = 0; u < FS_GROUP; ++u) {
          cur[u][0] = nxt[u][0];
          cur[u][1] = nxt[u][1];
        }
      }
    }
  }
  __syncthreads();

  // ---- C. Top-K of the rescored entries -------------------------------------
  {
    const int n = 8 * K;
    const int pw = 64 * PER2 * wv + lane;
    uint32_t key[PER2];
#pragma unroll
    for (int u = 0; u < PER2; ++u) key[u] = select_key(sc[pw + 64 * u < n ? pw + 64 * u : 0]);
#pragma unroll
    for (int u = 0; u < PER2; ++u) key[u] = pw + 64 * u < n ? key[u] : 0u;
    const uint32_t n_sel = block_select<FS_THREADS, PER2>(s, key, (uint32_t)K, [&](int p, uint32_t, uint32_t slot) {
      a.idx[q * K + slot] = 8 * top[p >> 3] + (p & 7);
    });
    for (int j = (int)n_sel + tid; j < K; j += FS_THREADS) a.idx[q * K + j] = -1;
  }
}

bool full_select_supported(int64_t nblk, int32_t nb, int32_t k) {
  return nblk <= SEL_CHUNK_MAX && nb <= SEL_POOL_MAX && k <= FS_KMAX && nb >= k;
}

hipError_t launch_full_select(const float* block_max, int64_t nblk, int64_t Q, int32_t nb, int32_t* pool,
                              int32_t k, int32_t* idx, const uint8_t* q_fp8, const float* w, const int32_t* q_pos,
                              int64_t q_per_seq, const uint8_t* k_fp8, int64_t k_rows, int64_t n_entries,
                              hipStream_t st) {
  if (Q == 0) return hipSuccess;
  FullSelArgs a{block_max, nblk, nb, pool, k, idx, q_fp8, w, q_pos, q_per_seq, k_fp8, k_rows, n_entries};
  const dim3 grid(1, (unsigned)Q), blk(FS_THREADS);
  const bool big1 = nblk > FS_THREADS * 16, big2 = 8 * (int64_t)k > FS_THREADS * 4;
  if (!big1 && !big2) hipLaunchKernelGGL((full_select_kernel<16, 4>), grid, blk, 0, st, a);
  else if (!big1) hipLaunchKernelGGL((full_select_kernel<16, 8>), grid, blk, 0, st, a);
  else if (!big2) hipLaunchKernelGGL((full_select_kernel<32, 4>), grid, blk, 0, st, a);
  else hipLaunchKernelGGL((full_select_kernel<32, 8>), grid, blk, 0, st, a);
  return hipGetLastError();
}

}  // namespace csa

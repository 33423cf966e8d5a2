// Fused Full-layer selection: the block pool, then the Top-K by rescoring
// only the entries of the best blocks.
//
// "DeepSeek-V4.1 架构解析" §02: a Full layer scores every causally visible entry, keeps the
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
// One block per query (1,024 threads, or 512 for many queries with top_k <=
// 512: about 68 KB of LDS, so two blocks share a compute unit and overlap
// each other's barriers and memory waits):
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
  const float* scores;      // [Q, n_entries] written by the scan, or null
  // split selection (decode batches): the pool kernel writes the chosen
  // blocks to top_out [Q, K] and zeroes ticket [Q]; full_rescore_kernel
  // rescores them in several blocks per query, publishes the scores in
  // sc_out [Q, 8 K] and the last block of a query selects the Top-K
  int32_t* top_out;
  int32_t* ticket;
  float* sc_out;
};

// Rescore the entries of blocks list[0 .. n) of query q (-1 = no block)
// with the scan's own arithmetic (the same fragments and fp32 sums, so the
// same bits): out[8 i + e] = score of entry 8 list[i] + e, -inf when absent
// or not visible.  Every wave of the NW-wave block calls it with its own LDS
// staging slot; n <= 64 NW.
//
// Wave wv takes fragments f = wv + NW i, i < n_mine, each two of the blocks
// (halves).  Lane L < 2 n_mine keeps half L's block: its number of visible
// entries (cnt) and the block to read (row 0's block when it has none, so
// every load reads existing rows); every half reads them back as
// wave-uniform values.  Loads are unconditional and the groups of FS_GROUP
// fragments alternate between two register sets, so no register with a load
// in flight is copied.  32-bit: entries < 2^30.
template <int NW>
__device__ __forceinline__ void rescore_blocks(const FullSelArgs& a, int64_t q, const int32_t* list, int n,
                                               float* out, uint4* stage, int wv, int lane) {
  const int64_t seq = q / a.q_per_seq;
  const int nv_pos = visible_count(a.q_pos[q]);
  const int64_t nv = nv_pos < a.n_entries ? nv_pos : a.n_entries;
  const int n_frag = (n + 1) / 2;   // two blocks per 16-entry fragment
  if (nv == 0) {   // nothing visible: every slot is empty (and no row may be read)
    for (int i = 64 * wv + lane; i < 16 * n_frag; i += 64 * NW) out[i] = -__builtin_huge_valf();
    return;
  }
  const int rowa = lane & 15;
  const Frag16 afrag = load_qfrag(a.q_fp8, q, rowa, rowa < IH, lane);
  float w4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) w4[r] = (lane < 32) ? a.w[q * IH + 4 * (lane >> 4) + r] : 0.f;
  const uint8_t* kbase = a.k_fp8 + seq * a.k_rows * ID;
  constexpr int FS_GROUP = 4;
  const int n_mine = (n_frag - wv + NW - 1) / NW;   // <= 32
  int my_cnt = 0, my_blkc = 0;
  {
    const int f = wv + NW * (lane >> 1), bi = 2 * f + (lane & 1);
    const int32_t blk = ((lane >> 1) < n_mine && bi < n) ? list[bi] : -1;
    // a block past the visible entries (or any id outside them) has no
    // visible entry; the test comes before the multiply, so 8 * blk <= nv
    const bool in_range = blk >= 0 && blk <= ((int)nv >> 3);
    const int rem = in_range ? (int)nv - 8 * blk : 0;
    my_cnt = rem <= 0 ? 0 : (rem >= 8 ? 8 : rem);
    my_blkc = my_cnt > 0 ? blk : 0;
  }
  const int lrow_k = lane >> 3;
  const uint32_t off_row[2] = {(uint32_t)(lrow_k * ID + 16 * stage_chunk(lane, 0)),
                               (uint32_t)(lrow_k * ID + 16 * stage_chunk(lane, 1))};
  const uint32_t off_zero[2] = {(uint32_t)(16 * stage_chunk(lane, 0)), (uint32_t)(16 * stage_chunk(lane, 1))};
  auto load_group = [&](int grp, uint4 (&v)[FS_GROUP][2]) {
#pragma unroll
    for (int u = 0; u < FS_GROUP; ++u) {
      const int i = grp * FS_GROUP + u;   // may pass n_mine: reads row 0, never used
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int hl = (2 * i + h) & 63;
        const int cnt = __builtin_amdgcn_readlane(my_cnt, hl);
        const uint8_t* base = kbase + (int64_t)__builtin_amdgcn_readlane(my_blkc, hl) * (8 * ID);
        v[u][h] = load16<false>(base + (lrow_k < cnt ? off_row[h] : off_zero[h]));
      }
    }
  };
  auto compute_group = [&](int grp, const uint4 (&v)[FS_GROUP][2]) {
#pragma unroll
    for (int u = 0; u < FS_GROUP; ++u) {
      const int i = grp * FS_GROUP + u;
      if (i >= n_mine) break;   // wave-uniform
      const int f = wv + NW * i;
      __builtin_amdgcn_wave_barrier();
      stage[lane] = v[u][0];
      stage[64 + lane] = v[u][1];
      __builtin_amdgcn_wave_barrier();
      const f32x4 acc = frag_mma(afrag, to_frag(read_staged(stage, lane)));
      const float sco = head_sum(acc, w4);
      // lane m < 16 holds column m: entry m % 8 of half m / 8, valid when
      // m % 8 is below that half's visible count (<= 8): bit m of a
      // wave-uniform mask built on the scalar unit
      const uint32_t c0 = __builtin_amdgcn_readlane(my_cnt, (2 * i) & 63);
      const uint32_t c1 = __builtin_amdgcn_readlane(my_cnt, (2 * i + 1) & 63);
      const uint32_t m16 = ((1u << c0) - 1u) | (((1u << c1) - 1u) << 8);
      if (lane < 16) out[16 * f + lane] = __builtin_amdgcn_inverse_ballot_w64((uint64_t)m16) ? sco : -__builtin_huge_valf();
    }
  };
  const int n_groups = (n_mine + FS_GROUP - 1) / FS_GROUP;
  uint4 ra[FS_GROUP][2], rb[FS_GROUP][2];
  load_group(0, ra);
  for (int grp = 0; grp < n_groups; grp += 2) {
    if (grp + 1 < n_groups) load_group(grp + 1, rb);
    compute_group(grp, ra);
    if (grp + 2 < n_groups) load_group(grp + 2, ra);
    if (grp + 1 < n_groups) compute_group(grp + 1, rb);
  }
}

// NT threads; block maxima per thread; rescored entries per thread; top_k
// bound (8 KMAX rescored scores in LDS).  The pool (phase A) and the key
// staging (phase B) are never live together and share their LDS.
template <int NT, int PER, int PER2, int KMAX>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void full_select_kernel(FullSelArgs a) {
  constexpr int FS_WAVES = NT / 64;
  __shared__ SelShared s;
  __shared__ union {
    int32_t pool[SEL_POOL_MAX];
    uint4 stage_all[FS_WAVES][128];
  } ps;
  __shared__ int32_t top[KMAX];
  __shared__ float sc[8 * KMAX];
  int32_t* pool = ps.pool;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.y;
  const int NB = a.NB, K = a.K;

  // ---- split selection with a pool (gridDim.x == 2): block x = 0 selects the
  // pool (for the Reindex layers), block x = 1 the top_k best blocks straight
  // from all the maxima (the same blocks as the best of the pool: the pool
  // holds the NB best blocks under the same order), so neither waits for the
  // other.  Block 1 then hands the blocks to full_rescore_kernel (top_out),
  // or, when the scan wrote every score, goes on to phases B and C itself.
  if (gridDim.x == 2) {
    const int pw = 64 * PER * wv + lane;
    uint32_t key[PER];
    load_keys<PER>(a.block_max + q * a.nblk, pw, (int)a.nblk, key);
    if (blockIdx.x == 0) {
      const uint32_t n_pool = block_select<NT, PER>(s, key, (uint32_t)NB, [&](int p, uint32_t, uint32_t slot) {
        if (a.pool_out) a.pool_out[q * NB + slot] = p;
      });
      if (a.pool_out)
        for (int j = (int)n_pool + tid; j < NB; j += NT) a.pool_out[q * NB + j] = -1;
      return;
    }
    if (a.top_out) {
      const uint32_t n_top = block_select<NT, PER>(s, key, (uint32_t)K, [&](int p, uint32_t, uint32_t slot) {
        a.top_out[q * K + slot] = p;
      });
      for (int j = (int)n_top + tid; j < K; j += NT) a.top_out[q * K + j] = -1;
      if (tid == 0) a.ticket[q] = 0;
      return;
    }
    const uint32_t n_top = block_select<NT, PER>(s, key, (uint32_t)K, [&](int p, uint32_t, uint32_t slot) {
      top[slot] = p;
    });
    for (int j = (int)n_top + tid; j < K; j += NT) top[j] = -1;
  } else {
  // ---- A. pool, and the top_k blocks ------------------------------------------
    const int pw = 64 * PER * wv + lane;
    const float* row = a.block_max + q * a.nblk;
    {
      uint32_t key[PER];
      load_keys<PER>(row, pw, (int)a.nblk, key);
      const uint32_t n_pool = block_select<NT, PER>(s, key, (uint32_t)NB, [&](int p, uint32_t, uint32_t slot) {
        pool[slot] = p;
        if (a.pool_out) a.pool_out[q * NB + slot] = p;
      });
      for (int j = (int)n_pool + tid; j < NB; j += NT) {
        pool[j] = -1;
        if (a.pool_out) a.pool_out[q * NB + j] = -1;
      }
    }
    if (NB > K) {
      // the top_k blocks are among the pool: select them from the pool's own
      // block maxima (pool order is id order, so ties still go to lower ids)
      __syncthreads();   // pool is complete
      constexpr int PP = SEL_POOL_MAX / NT;
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
      const uint32_t n_top = block_select<NT, PP>(s, key, (uint32_t)K, [&](int i, uint32_t, uint32_t slot) {
        top[slot] = pool[i];
      });
      for (int j = (int)n_top + tid; j < K; j += NT) top[j] = -1;
    } else {
      __syncthreads();   // pool is complete
      for (int j = tid; j < K; j += NT) top[j] = pool[j];
    }
  }
  __syncthreads();
  if (a.top_out) {   // (one block per query) the chosen blocks go to full_rescore_kernel
    for (int j = tid; j < K; j += NT) a.top_out[q * K + j] = top[j];
    if (tid == 0) a.ticket[q] = 0;
    return;
  }

  // ---- B. the scores of the top_k blocks' entries ----------------------------
  if (a.scores) {
    // decode batches: the scan wrote every column's score (-inf past the
    // visible entries), so gather the 8 scores of each chosen block -- every
    // load issued before any is used, each from an existing column
    constexpr int GPT = 8 * KMAX / NT;   // slots per thread
    const float* srow = a.scores + q * a.n_entries;
    float v[GPT];
    bool ok[GPT];
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int slot = tid + NT * u;   // block slot >> 3, entry slot & 7
      const int i = slot >> 3;
      const int32_t b = i < K ? top[i] : -1;
      const int64_t col = 8 * (int64_t)b + (slot & 7);
      ok[u] = b >= 0 && col < a.n_entries;
    }
    if (a.n_entries > 0) {   // block-uniform: an empty row has nothing to read
#pragma unroll
      for (int u = 0; u < GPT; ++u) {
        const int slot = tid + NT * u;
        const int32_t b = (slot >> 3) < K ? top[slot >> 3] : -1;
        v[u] = srow[ok[u] ? 8 * (int64_t)b + (slot & 7) : 0];
      }
    }
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int slot = tid + NT * u;
      if (slot < 8 * K) sc[slot] = ok[u] ? v[u] : -__builtin_huge_valf();
    }
  } else {
    rescore_blocks<FS_WAVES>(a, q, top, K, sc, ps.stage_all[wv], wv, lane);
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
    const uint32_t n_sel = block_select<NT, PER2>(s, key, (uint32_t)K, [&](int p, uint32_t, uint32_t slot) {
      a.idx[q * K + slot] = 8 * top[p >> 3] + (p & 7);
    });
    for (int j = (int)n_sel + tid; j < K; j += NT) a.idx[q * K + j] = -1;
  }
}

// ---------------------------------------------------------------------------
// Split Full-layer selection, second kernel: block (r, q) of 16 waves
// rescores the chosen blocks r P .. r P + P - 1 of query q (P = ceil(K / R),
// R = gridDim.x), so one query's 512 KiB of key gathers spread over R
// compute units instead of one.  The scores go out as device-coherent
// stores (written through to memory, sc1), each thread waits for its own
// stores, and thread 0 then takes the query's ticket (an agent-scope atomic
// add, which the pool kernel zeroed).  The block that draws the last ticket
// reads every score back with device-coherent loads and selects the Top-K,
// ties to the lower entry; no fence that writes back a whole L2 is needed.
constexpr int FR_THREADS = 1024;
constexpr int FR_WAVES = FR_THREADS / 64;
constexpr int FR_MAX_BLOCKS = 64 * FR_WAVES;   // blocks one rescoring block takes (rescore_blocks' bound)

template <int PER2>
__global__ __launch_bounds__(FR_THREADS) void full_rescore_kernel(FullSelArgs a) {
  __shared__ SelShared s;
  __shared__ int32_t top[FS_KMAX];
  __shared__ float sc[8 * FR_MAX_BLOCKS];
  __shared__ uint4 stage_all[FR_WAVES][128];
  __shared__ int32_t last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.y;
  const int K = a.K, R = gridDim.x, r = blockIdx.x;
  const int per = (K + R - 1) / R;
  const int b0 = r * per, nb = (b0 + per < K ? b0 + per : K) - b0;   // this block's slots of top
  for (int j = tid; j < K; j += FR_THREADS) top[j] = a.top_out[q * K + j];
  __syncthreads();
  if (nb > 0) rescore_blocks<FR_WAVES>(a, q, top + b0, nb, sc, stage_all[wv], wv, lane);
  __syncthreads();
  float* srow = a.sc_out + q * (int64_t)(8 * K);
  for (int i = tid; i < 8 * nb; i += FR_THREADS)
    __hip_atomic_store(srow + 8 * b0 + i, sc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);   // this thread's stores have reached memory
  __syncthreads();
  if (tid == 0) last = __hip_atomic_fetch_add(a.ticket + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (last != R - 1) return;   // block-uniform: another block selects

  // ---- the last block: Top-K of the query's 8 K scores ----------------------------
  const int n = 8 * K;
  const int pw = 64 * PER2 * wv + lane;
  uint32_t key[PER2];
#pragma unroll
  for (int u = 0; u < PER2; ++u) {
    const int p = pw + 64 * u;
    key[u] = select_key(__hip_atomic_load(srow + (p < n ? p : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
#pragma unroll
  for (int u = 0; u < PER2; ++u) key[u] = pw + 64 * u < n ? key[u] : 0u;
  const uint32_t n_sel = block_select<FR_THREADS, PER2>(s, key, (uint32_t)K, [&](int p, uint32_t, uint32_t slot) {
    a.idx[q * K + slot] = 8 * top[p >> 3] + (p & 7);
  });
  for (int j = (int)n_sel + tid; j < K; j += FR_THREADS) a.idx[q * K + j] = -1;
}

// Block maxima per thread: the fewest of 4, 8, 16, 24, 32 that hold nblk (a
// row's padding slots still cost every per-key step of the selection).
static int fs_keys_per_thread(int64_t nblk, int nt) {
  const int per[5] = {4, 8, 16, 24, 32};
  for (int i = 0; i < 4; ++i)
    if ((int64_t)nt * per[i] >= nblk) return per[i];
  return 32;
}

template <int NT, int PER2, int KMAX>
void launch_full_select_per(int per, dim3 grid, hipStream_t st, const FullSelArgs& a) {
  switch (per) {
    case 4: hipLaunchKernelGGL((full_select_kernel<NT, 4, PER2, KMAX>), grid, dim3(NT), 0, st, a); break;
    case 8: hipLaunchKernelGGL((full_select_kernel<NT, 8, PER2, KMAX>), grid, dim3(NT), 0, st, a); break;
    case 16: hipLaunchKernelGGL((full_select_kernel<NT, 16, PER2, KMAX>), grid, dim3(NT), 0, st, a); break;
    case 24: hipLaunchKernelGGL((full_select_kernel<NT, 24, PER2, KMAX>), grid, dim3(NT), 0, st, a); break;
    default: hipLaunchKernelGGL((full_select_kernel<NT, 32, PER2, KMAX>), grid, dim3(NT), 0, st, a); break;
  }
}

bool full_select_supported(int64_t nblk, int32_t nb, int32_t k) {
  return nblk <= SEL_CHUNK_MAX && nb <= SEL_POOL_MAX && k <= FS_KMAX && nb >= k;
}

hipError_t launch_full_select(const float* block_max, int64_t nblk, int64_t Q, int32_t nb, int32_t* pool,
                              int32_t k, int32_t* idx, const uint8_t* q_fp8, const float* w, const int32_t* q_pos,
                              int64_t q_per_seq, const uint8_t* k_fp8, int64_t k_rows, int64_t n_entries,
                              const float* scores, void* split_ws, hipStream_t st) {
  if (Q == 0) return hipSuccess;
  FullSelArgs a{block_max, nblk, nb, pool, k, idx, q_fp8, w, q_pos, q_per_seq, k_fp8, k_rows, n_entries, scores,
                nullptr, nullptr, nullptr};
  int R = 0;
  if (split_ws) {
    // blocks per query: about one per compute unit in all, each rescoring
    // at most FR_MAX_BLOCKS chosen blocks
    R = (int)((256 + Q - 1) / Q);
    R = R > 16 ? 16 : R;
    const int r_min = (k + FR_MAX_BLOCKS - 1) / FR_MAX_BLOCKS;
    R = R < r_min ? r_min : R;
    char* p = reinterpret_cast<char*>(split_ws);
    a.top_out = reinterpret_cast<int32_t*>(p);
    a.ticket = reinterpret_cast<int32_t*>(p + full_split_top_bytes(Q, k));
    a.sc_out = reinterpret_cast<float*>(p + full_split_top_bytes(Q, k) + full_split_ticket_bytes(Q));
  }
  // decode batches with a pool: two blocks per query (pool, best blocks),
  // whether the best blocks are then rescored or their scores gathered
  const dim3 grid(nb > k && (split_ws || (scores && Q < 512)) ? 2 : 1, (unsigned)Q);
  // many queries: 512-thread blocks, two per compute unit (top_k <= 512,
  // nblk <= 16,384); a few queries: 1,024 threads, the shortest block
  if (Q >= 512 && k <= 512 && nblk <= 512 * 32) {
    launch_full_select_per<512, 8, 512>(fs_keys_per_thread(nblk, 512), grid, st, a);
    return hipGetLastError();
  }
  if (8 * (int64_t)k <= FS_THREADS * 4)
    launch_full_select_per<FS_THREADS, 4, FS_KMAX>(fs_keys_per_thread(nblk, FS_THREADS), grid, st, a);
  else
    launch_full_select_per<FS_THREADS, 8, FS_KMAX>(fs_keys_per_thread(nblk, FS_THREADS), grid, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split_ws) return e;
  const dim3 g2((unsigned)R, (unsigned)Q);
  if (8 * (int64_t)k <= FR_THREADS * 4)
    hipLaunchKernelGGL(full_rescore_kernel<4>, g2, dim3(FR_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(full_rescore_kernel<8>, g2, dim3(FR_THREADS), 0, st, a);
  return hipGetLastError();
}

size_t full_split_top_bytes(int64_t Q, int32_t k) { return ((size_t)Q * k * 4 + 255) / 256 * 256; }
size_t full_split_ticket_bytes(int64_t Q) { return ((size_t)Q * 4 + 255) / 256 * 256; }
size_t full_split_workspace_bytes(int64_t Q, int32_t k) {
  return full_split_top_bytes(Q, k) + full_split_ticket_bytes(Q) + (size_t)Q * 8 * k * 4;
}

}  // namespace csa

// Top-K selection and the hierarchical block pool.
//
// "DeepSeek-V4.1 架构解析" §02: the first Full layer picks the Top-512 over every visible position,
// then ranks 8-position blocks by their largest score and keeps 2,048 of them
// (16,384 candidates) for the Reindex layers.  Equal scores go to the lower
// column (and so the lower entry id); -inf and NaN columns are never selected.
//
// One block of NT threads selects the K best of up to NT * PER keys held in
// registers, PER per thread (lane l of wave v holds positions
// 64 PER v + 64 u + l, u < PER, so that every load is one contiguous run):
//   1. block-reduce the largest and smallest valid value and the valid count;
//   2. histogram the values into SEL_BINS bins linear in value between the two
//      (a monotone map, so every key of a lower bin beats every key of a
//      higher one) and scan it to find the bin holding the K-th largest key;
//   3. find that key T exactly among the bin's keys only: pairwise ranking
//      when the bin is small, else a three-digit radix select over the keys
//      of the bin; also how many keys equal to T are still needed;
//   4. compact in position order (a block scan of per-wave counts, then wave
//      ballots), which keeps the output ascending and gives ties to the lower
//      positions.
// Rows of 8K+ keys first narrow the keys to a sampled lower bound of the K-th
// largest (block_select), so that steps 1-4 run over about 1.5 K candidates.
// Longer rows are cut into chunks whose K best are kept as candidates (the
// global K best are among them) and selected again.  A Full layer runs the
// block pool and the Top-K among the pooled blocks' entries in one kernel.
#include "common.h"
#include "kernels.h"
#include "select_core.h"

namespace csa {

using namespace sel;

// MODE 0: keys come from float scores [Q, ncols] (column = position);
// MODE 1: keys / columns come from candidate arrays [Q, n_in];
// MODE 2: positions are the entries of the blocks listed in
//   col_blocks [Q, nblk_map] (ascending, -1 padded): position i is entry
//   8 * col_blocks[q, i / 8] + i % 8 of scores [Q, ncols]; n_in = 8 * nblk_map.
// FINAL: write ids ascending to idx [Q, K] (with col_blocks, MODE 0 / 1 map
// the column through the blocks); otherwise write the chunk's K best (key,
// column) pairs ascending to out_keys / out_cols [Q, gridDim.x * K] (MODE 2
// writes entry ids as the columns).  One block per (chunk of NT PER keys, row).
template <int MODE, bool FINAL, int NT, int PER>
__global__ __launch_bounds__(NT) void select_kernel(
    const float* __restrict__ scores, int64_t ncols, const uint32_t* __restrict__ cand_keys,
    const int32_t* __restrict__ cand_cols, int64_t n_in, const int32_t* __restrict__ col_blocks,
    int64_t nblk_map, int32_t K, int32_t* __restrict__ idx, uint32_t* __restrict__ out_keys,
    int32_t* __restrict__ out_cols) {
  __shared__ SelShared s;
  // The chunk's slice of col_blocks (MODE 0 with col_blocks, MODE 2), staged
  // while the keys load, so that writing an id reads LDS instead of waiting
  // on a global load after the selection.
  constexpr int MAPN = MODE == 1 ? 1 : NT * PER / 8;
  __shared__ int32_t bmap[MAPN];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.y;
  const int64_t total = MODE == 0 ? ncols : n_in;
  const int64_t start = (int64_t)blockIdx.x * (NT * PER);
  const int n = (int)((total - start) < NT * PER ? (total - start) : NT * PER);
  const int pw = 64 * PER * wv + lane;       // position of key[u] is pw + 64 u
  const bool staged = MODE != 1 && col_blocks != nullptr;
  if (staged) {
    // blocks start / 8 .. of the row (start is a multiple of 8); entries of
    // the chunk past the row's blocks are never selected
    const int64_t b0 = start >> 3;
    const int nb = (int)((nblk_map - b0) < MAPN ? (nblk_map - b0) : MAPN);
    for (int i = tid; i < nb; i += NT) bmap[i] = col_blocks[q * nblk_map + b0 + i];
  }

  uint32_t key[PER];   // 0 = not selectable
  if (MODE == 0) {
    load_keys<PER>(scores + q * ncols + start, pw, n, key);
  } else if (MODE == 2) {
    const int32_t* map = col_blocks + q * nblk_map + (start >> 3);   // start is a multiple of 8
    gather_keys<PER>(scores + q * ncols, ncols, pw, n, [&](int slot) { return map[slot]; }, key);
  } else {
    load_raw_keys<PER>(cand_keys + q * n_in + start, pw, n, key);
  }

  const uint32_t n_sel = block_select<NT, PER>(s, key, (uint32_t)K, [&](int p, uint32_t k, uint32_t slot) {
    const int64_t pos = start + p;
    int64_t col;
    if (MODE == 0) col = pos;
    else if (MODE == 1) col = cand_cols[q * n_in + pos];
    else col = 8 * (int64_t)bmap[p >> 3] + (pos & 7);
    if (FINAL) {
      int64_t id = col;
      if (MODE == 0 && col_blocks) id = 8 * (int64_t)bmap[p >> 3] + (col & 7);
      else if (MODE == 1 && col_blocks) id = 8 * (int64_t)col_blocks[q * nblk_map + (col >> 3)] + (col & 7);
      idx[q * K + slot] = (int32_t)id;
    } else {
      const int64_t o = (q * gridDim.x + blockIdx.x) * (int64_t)K + slot;
      out_keys[o] = k;
      out_cols[o] = (int32_t)col;
    }
  });
  for (int j = (int)n_sel + tid; j < K; j += NT) {
    if (FINAL) {
      idx[q * K + j] = -1;
    } else {
      const int64_t o = (q * gridDim.x + blockIdx.x) * (int64_t)K + j;
      out_keys[o] = 0u;
      out_cols[o] = -1;
    }
  }
}

// Full layer, one block per row: the NB blocks with the largest block max
// (block_max [Q, nblk], nblk <= NT PER) -> pool [Q, NB] (ascending, -1
// padded; may be null), then the K best of the pooled blocks' entries
// (scores [Q, ncols]; 8 NB <= NT PER2) -> idx [Q, K] ascending, -1 padded.
template <int NT, int PER, int PER2>
__global__ __launch_bounds__(NT) void pool_topk_kernel(
    const float* __restrict__ block_max, int64_t nblk, const float* __restrict__ scores, int64_t ncols,
    int32_t NB, int32_t* __restrict__ pool_out, int32_t K, int32_t* __restrict__ idx) {
  __shared__ SelShared s;
  __shared__ int32_t pool[SEL_POOL_MAX];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.y;
  {
    const int pw = 64 * PER * wv + lane;
    const float* row = block_max + q * nblk;
    uint32_t key[PER];
    load_keys<PER>(row, pw, (int)nblk, key);
    const uint32_t n_sel = block_select<NT, PER>(s, key, (uint32_t)NB, [&](int p, uint32_t, uint32_t slot) {
      pool[slot] = p;
      if (pool_out) pool_out[q * NB + slot] = p;
    });
    for (int j = (int)n_sel + tid; j < NB; j += NT) {
      pool[j] = -1;
      if (pool_out) pool_out[q * NB + j] = -1;
    }
  }
  __syncthreads();
  const int pw = 64 * PER2 * wv + lane;
  const int n = 8 * NB;
  const float* row = scores + q * ncols;
  uint32_t key[PER2];
  gather_keys<PER2>(row, ncols, pw, n, [&](int slot) { return pool[slot]; }, key);
  const uint32_t n_sel = block_select<NT, PER2>(s, key, (uint32_t)K, [&](int p, uint32_t, uint32_t slot) {
    idx[q * K + slot] = 8 * pool[p >> 3] + (p & 7);
  });
  for (int j = (int)n_sel + tid; j < K; j += NT) idx[q * K + j] = -1;
}

// Block maxima over aligned 8-column blocks (-inf entries ignored).
__global__ __launch_bounds__(256) void block_max_kernel(const float* __restrict__ v, int64_t Q,
                                                        int64_t ncols, float* __restrict__ bm) {
  int64_t nblk = (ncols + 7) >> 3;
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= Q * nblk) return;
  int64_t q = t / nblk, b = t % nblk;
  float m = -__builtin_huge_valf();
  for (int j = 0; j < 8; ++j) {
    int64_t c = 8 * b + j;
    if (c < ncols) m = fmaxf(m, v[q * ncols + c]);
  }
  bm[t] = m;
}

namespace {
// Block shapes: 1024 threads (four waves per SIMD hide the latency of each
// step) with 16 keys each for rows up to 16K keys, 32 up to 32K.  Many rows
// (prefill chunks) are throughput-bound instead: single selections then use
// 512 threads with 32 keys each (about 80 registers, so three blocks, 24
// waves, share a compute unit; 256 threads with 64 keys need ~150 registers
// and spill scalar registers heavily, three blocks of 4 waves, and took 1.5x
// as long).
constexpr int SEL_NT = 1024, SEL_PER_S = 16, SEL_PER_L = 32;
constexpr int SEL_NT_T = 512, SEL_PER_T = 32;
constexpr int64_t SEL_MANY_ROWS = 1024;
static_assert(SEL_NT * SEL_PER_L == SEL_CHUNK_MAX, "block shape");

int64_t chunks_of(int64_t n) { return (n + SEL_CHUNK_MAX - 1) / SEL_CHUNK_MAX; }

// Candidate-buffer length per row needed by the multi-stage selection.
int64_t cand_len(int64_t ncols, int32_t k) {
  int64_t c = chunks_of(ncols);
  if (c <= 1) return 0;
  return c * (int64_t)k;
}

// One block per row over n <= SEL_CHUNK_MAX keys.
template <int MODE>
void launch_single(int64_t n, int64_t Q, const float* scores, int64_t ncols, const uint32_t* ck,
                   const int32_t* cc, int64_t n_in, const int32_t* col_blocks, int64_t nblk_map, int32_t k,
                   int32_t* idx, hipStream_t st) {
  if (Q >= SEL_MANY_ROWS && n <= SEL_NT_T * SEL_PER_T)
    hipLaunchKernelGGL((select_kernel<MODE, true, SEL_NT_T, SEL_PER_T>), dim3(1, (unsigned)Q), dim3(SEL_NT_T), 0,
                       st, scores, ncols, ck, cc, n_in, col_blocks, nblk_map, k, idx, nullptr, nullptr);
  else if (n <= SEL_NT * SEL_PER_S)
    hipLaunchKernelGGL((select_kernel<MODE, true, SEL_NT, SEL_PER_S>), dim3(1, (unsigned)Q), dim3(SEL_NT), 0,
                       st, scores, ncols, ck, cc, n_in, col_blocks, nblk_map, k, idx, nullptr, nullptr);
  else
    hipLaunchKernelGGL((select_kernel<MODE, true, SEL_NT, SEL_PER_L>), dim3(1, (unsigned)Q), dim3(SEL_NT), 0,
                       st, scores, ncols, ck, cc, n_in, col_blocks, nblk_map, k, idx, nullptr, nullptr);
}

// Chunk candidates (keys0 / cols0, n_in per row) -> final ids.
hipError_t merge_candidates(int64_t Q, int64_t n_in, int32_t k, uint32_t* keys0, int32_t* cols0,
                            uint32_t* keys1, int32_t* cols1, const int32_t* col_blocks, int64_t nblk_map,
                            int32_t* idx, hipStream_t st) {
  hipError_t e;
  while (chunks_of(n_in) > 1) {
    const int64_t c2 = chunks_of(n_in);
    hipLaunchKernelGGL((select_kernel<1, false, SEL_NT, SEL_PER_L>), dim3((unsigned)c2, (unsigned)Q),
                       dim3(SEL_NT), 0, st, nullptr, 0, keys0, cols0, n_in, nullptr, 0, k, nullptr, keys1,
                       cols1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint32_t* tk = keys0; keys0 = keys1; keys1 = tk;
    int32_t* tc = cols0; cols0 = cols1; cols1 = tc;
    n_in = c2 * k;
  }
  launch_single<1>(n_in, Q, nullptr, 0, keys0, cols0, n_in, col_blocks, nblk_map, k, idx, st);
  return hipGetLastError();
}
}  // namespace

size_t topk_workspace_bytes(int64_t Q, int64_t ncols, int32_t k) {
  const int64_t len = cand_len(ncols, k);
  // two ping-pong candidate buffers of (key, column) pairs
  return (size_t)(2 * Q * len) * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_topk(const float* scores, int64_t Q, int64_t ncols, const int32_t* col_blocks,
                       int32_t k, int32_t* idx, void* ws, hipStream_t st) {
  if (Q == 0) return hipSuccess;
  const int64_t nblk_map = (ncols + 7) >> 3;
  const int64_t c = chunks_of(ncols);
  if (c <= 1) {
    launch_single<0>(ncols, Q, scores, ncols, nullptr, nullptr, 0, col_blocks, nblk_map, k, idx, st);
    return hipGetLastError();
  }
  const int64_t len = cand_len(ncols, k);
  uint32_t* keys0 = reinterpret_cast<uint32_t*>(ws);
  int32_t* cols0 = reinterpret_cast<int32_t*>(keys0 + Q * len);
  uint32_t* keys1 = reinterpret_cast<uint32_t*>(cols0 + Q * len);
  int32_t* cols1 = reinterpret_cast<int32_t*>(keys1 + Q * len);
  hipLaunchKernelGGL((select_kernel<0, false, SEL_NT, SEL_PER_L>), dim3((unsigned)c, (unsigned)Q),
                     dim3(SEL_NT), 0, st, scores, ncols, nullptr, nullptr, 0, nullptr, 0, k, nullptr, keys0,
                     cols0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return merge_candidates(Q, c * k, k, keys0, cols0, keys1, cols1, col_blocks, nblk_map, idx, st);
}

size_t topk_gather_workspace_bytes(int64_t Q, int64_t nmap, int32_t k) {
  return topk_workspace_bytes(Q, 8 * nmap, k);
}

// K best entries among the entries of the listed blocks (MODE 2), ascending ids.
hipError_t launch_topk_gather(const float* scores, int64_t Q, int64_t ncols, const int32_t* blocks,
                              int64_t nmap, int32_t k, int32_t* idx, void* ws, hipStream_t st) {
  if (Q == 0) return hipSuccess;
  const int64_t n = 8 * nmap;
  const int64_t c = chunks_of(n);
  if (c <= 1) {
    launch_single<2>(n, Q, scores, ncols, nullptr, nullptr, n, blocks, nmap, k, idx, st);
    return hipGetLastError();
  }
  const int64_t len = cand_len(n, k);
  uint32_t* keys0 = reinterpret_cast<uint32_t*>(ws);
  int32_t* cols0 = reinterpret_cast<int32_t*>(keys0 + Q * len);
  uint32_t* keys1 = reinterpret_cast<uint32_t*>(cols0 + Q * len);
  int32_t* cols1 = reinterpret_cast<int32_t*>(keys1 + Q * len);
  hipLaunchKernelGGL((select_kernel<2, false, SEL_NT, SEL_PER_L>), dim3((unsigned)c, (unsigned)Q),
                     dim3(SEL_NT), 0, st, scores, ncols, nullptr, nullptr, n, blocks, nmap, k, nullptr, keys0,
                     cols0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return merge_candidates(Q, c * k, k, keys0, cols0, keys1, cols1, nullptr, 0, idx, st);
}

size_t block_pool_workspace_bytes(int64_t Q, int64_t ncols, int32_t is_block_max, int32_t nb) {
  const int64_t nblk = is_block_max ? ncols : (ncols + 7) / 8;
  size_t bm = is_block_max ? 0 : (size_t)(Q * nblk) * sizeof(float);
  bm = (bm + 255) & ~(size_t)255;
  return bm + topk_workspace_bytes(Q, nblk, nb);
}

hipError_t launch_block_pool(const float* values, int32_t is_block_max, int64_t Q, int64_t ncols,
                             int32_t nb, int32_t* pool, void* ws, hipStream_t st) {
  if (Q == 0) return hipSuccess;
  const float* bm = values;
  int64_t nblk = ncols;
  char* rest = reinterpret_cast<char*>(ws);
  if (!is_block_max) {
    nblk = (ncols + 7) / 8;
    float* tmp = reinterpret_cast<float*>(ws);
    const int64_t tot = Q * nblk;
    hipLaunchKernelGGL(block_max_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, values, Q,
                       ncols, tmp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bm = tmp;
    const size_t used = ((size_t)tot * sizeof(float) + 255) & ~(size_t)255;
    rest += used;
  }
  return launch_topk(bm, Q, nblk, nullptr, nb, pool, rest, st);
}

size_t pool_topk_workspace_bytes(int64_t Q, int64_t nblk, int32_t nb, int32_t k) {
  if (nblk <= SEL_CHUNK_MAX && nb <= SEL_POOL_MAX) return 0;
  const size_t a = block_pool_workspace_bytes(Q, nblk, 1, nb);
  const size_t b = topk_gather_workspace_bytes(Q, nb, k);
  return a > b ? a : b;
}

hipError_t launch_pool_topk(const float* block_max, int64_t nblk, const float* scores, int64_t ncols,
                            int64_t Q, int32_t nb, int32_t* pool, int32_t k, int32_t* idx, void* ws,
                            hipStream_t st) {
  if (Q == 0) return hipSuccess;
  if (nblk <= SEL_CHUNK_MAX && nb <= SEL_POOL_MAX) {
    const dim3 grid(1, (unsigned)Q), blk(SEL_NT);
    const bool big1 = nblk > SEL_NT * SEL_PER_S, big2 = 8 * (int64_t)nb > SEL_NT * SEL_PER_S;
    if (!big1 && !big2)
      hipLaunchKernelGGL((pool_topk_kernel<SEL_NT, SEL_PER_S, SEL_PER_S>), grid, blk, 0, st, block_max, nblk,
                         scores, ncols, nb, pool, k, idx);
    else if (!big1)
      hipLaunchKernelGGL((pool_topk_kernel<SEL_NT, SEL_PER_S, SEL_PER_L>), grid, blk, 0, st, block_max, nblk,
                         scores, ncols, nb, pool, k, idx);
    else if (!big2)
      hipLaunchKernelGGL((pool_topk_kernel<SEL_NT, SEL_PER_L, SEL_PER_S>), grid, blk, 0, st, block_max, nblk,
                         scores, ncols, nb, pool, k, idx);
    else
      hipLaunchKernelGGL((pool_topk_kernel<SEL_NT, SEL_PER_L, SEL_PER_L>), grid, blk, 0, st, block_max, nblk,
                         scores, ncols, nb, pool, k, idx);
    return hipGetLastError();
  }
  // rows longer than one block: chunked block pool, then the gathered selection
  hipError_t e = launch_block_pool(block_max, 1, Q, nblk, nb, pool, ws, st);
  if (e != hipSuccess) return e;
  return launch_topk_gather(scores, Q, ncols, pool, nb, k, idx, ws, st);
}

}  // namespace csa

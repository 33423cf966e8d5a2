// Top-K selection and the hierarchical block pool.
//
// P3 §02: the first Full layer picks the Top-512 over every visible position,
// then ranks 8-position blocks by their largest score and keeps 2,048 of them
// (16,384 candidates) for the Reindex layers.  Equal scores go to the lower
// column (and so the lower entry id); -inf columns are never selected.
//
// One 1024-thread block selects the K best of up to SEL_CHUNK keys, 16 per
// thread in registers (lane l of wave v holds positions 1024 v + 64 u + l,
// u < 16, so that every load is one contiguous 256-byte run):
//   1. block-reduce the largest and smallest valid value and the valid count;
//   2. histogram the values into SEL_BINS bins linear in value between the two
//      (a monotone map, so every key of a lower bin beats every key of a
//      higher one) and scan it to find the bin holding the K-th largest key;
//   3. find that key T exactly among the bin's keys only (pairwise ranking
//      when the bin is small, else a three-digit radix select over it), and
//      how many keys equal to T are still needed;
//   4. compact in position order (a block scan of per-wave counts, then wave
//      ballots), which keeps the output ascending and gives ties to the lower
//      positions.
// Rows longer than SEL_CHUNK are cut into chunks; every chunk's K best are
// kept as candidates (the global K best are among them) and selected again.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int SEL_CHUNK = 16384;
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_PER = SEL_CHUNK / SEL_THREADS;      // keys per thread
constexpr int SEL_BINS = 2048;
constexpr int SEL_RANK_MAX = 256;                     // pairwise ranking up to this many keys

namespace {

struct SelShared {
  uint32_t hist[SEL_BINS];
  uint32_t cand[SEL_CHUNK];       // keys of the threshold bin
  uint32_t wred[3][SEL_WAVES];    // per-wave partials
  uint32_t n_cand, bstar, rem, T, take_eq;
};

// Value of a valid (non-zero) key: the inverse of select_key.
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Cross-lane steps on the DPP network (gfx9 controls: quad_perm, row_shr,
// row_mirror, row_half_mirror, row_bcast15, row_bcast31).  A lane whose source
// is outside the row mask keeps `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112,
              DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118, DPP_ROW_MIRROR = 0x140,
              DPP_ROW_HALF_MIRROR = 0x141, DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143;

// Inclusive prefix sum across the wave (lane 0 first).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<DPP_ROW_SHR1>(0u, v);
  v += dpp<DPP_ROW_SHR2>(0u, v);
  v += dpp<DPP_ROW_SHR4>(0u, v);
  v += dpp<DPP_ROW_SHR8>(0u, v);
  v += dpp<DPP_BCAST15, 0xA>(0u, v);
  v += dpp<DPP_BCAST31, 0xC>(0u, v);
  return v;
}

// Wave-wide max / min / sum, returned uniformly (the full result lands in lane 63).
template <int OP>   // 0 max, 1 min, 2 sum
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return OP == 0 ? (a > b ? a : b) : OP == 1 ? (a < b ? a : b) : a + b; };
  const uint32_t id = OP == 0 ? 0u : OP == 1 ? 0xFFFFFFFFu : 0u;
  v = f(v, dpp<DPP_XOR1>(id, v));
  v = f(v, dpp<DPP_XOR2>(id, v));
  v = f(v, dpp<DPP_ROW_HALF_MIRROR>(id, v));
  v = f(v, dpp<DPP_ROW_MIRROR>(id, v));
  v = f(v, dpp<DPP_BCAST15, 0xA>(id, v));
  v = f(v, dpp<DPP_BCAST31, 0xC>(id, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive block scan of v; *total = the block sum.  Two barriers.
__device__ __forceinline__ uint32_t block_excl_scan(SelShared& s, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) s.wred[0][wv] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t x = s.wred[0][w];
    before += w < wv ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Bin of a valid value: 0 holds the largest values.
__device__ __forceinline__ int value_bin(float v, float vmax, float inv) {
  if (inv == 0.0f) return 0;
  const float x = (vmax - v) * inv;
  return (int)fminf(x, (float)(SEL_BINS - 1));
}

// The rem-th largest of the n keys in s.cand (1 <= rem <= n) and how many
// keys equal to it are taken: exact three-digit radix select (11, 11, 10 bits).
__device__ void radix_select_cand(SelShared& s, int n, uint32_t rem) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  const int shifts[3] = {21, 10, 0};
  const uint32_t masks[3] = {0u, 0xFFE00000u, 0xFFFFFC00u};
  for (int pass = 0; pass < 3; ++pass) {
    for (int b = tid; b < SEL_BINS; b += SEL_THREADS) s.hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += SEL_THREADS) {
      const uint32_t k = s.cand[i];
      if ((k & masks[pass]) == prefix) atomicAdd(&s.hist[(k >> shifts[pass]) & (SEL_BINS - 1)], 1u);
    }
    __syncthreads();
    // thread t owns digits 2047 - 2t and 2046 - 2t (largest digits first)
    const uint32_t h0 = s.hist[SEL_BINS - 1 - 2 * tid], h1 = s.hist[SEL_BINS - 2 - 2 * tid];
    uint32_t total;
    const uint32_t excl = block_excl_scan(s, h0 + h1, &total);
    if (excl < rem && rem <= excl + h0 + h1) {
      const bool first = rem <= excl + h0;
      const uint32_t digit = first ? SEL_BINS - 1 - 2 * tid : SEL_BINS - 2 - 2 * tid;
      s.T = digit;
      s.rem = first ? rem - excl : rem - excl - h0;
    }
    __syncthreads();
    prefix |= s.T << shifts[pass];
    rem = s.rem;
    __syncthreads();
  }
  if (tid == 0) {
    s.T = prefix;
    s.take_eq = rem;
  }
}

}  // namespace

// MODE 0: keys come from float scores [Q, ncols] (column = position);
// MODE 1: keys / columns come from candidate arrays [Q, n_in];
// MODE 2: positions are the entries of the blocks listed in
//   col_blocks [Q, nblk_map] (ascending, -1 padded): position i is entry
//   8 * col_blocks[q, i / 8] + i % 8 of scores [Q, ncols]; n_in = 8 * nblk_map.
// FINAL: write ids ascending to idx [Q, K]; otherwise write the chunk's K
// best (key, column) pairs ascending to cand_out [Q, gridDim.x * K] (MODE 2
// writes entry ids as the columns).  One block per (chunk, row).
template <int MODE, bool FINAL>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const float* __restrict__ scores, int64_t ncols, const uint32_t* __restrict__ cand_keys,
    const int32_t* __restrict__ cand_cols, int64_t n_in, const int32_t* __restrict__ col_blocks,
    int64_t nblk_map, int32_t K, int32_t* __restrict__ idx, uint32_t* __restrict__ out_keys,
    int32_t* __restrict__ out_cols) {
  __shared__ SelShared s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.y;
  const int64_t total = MODE == 0 ? ncols : n_in;
  const int64_t start = (int64_t)blockIdx.x * SEL_CHUNK;
  const int n = (int)((total - start) < SEL_CHUNK ? (total - start) : SEL_CHUNK);
  const int pw = 1024 * wv + lane;       // position of key[u] is pw + 64 u

  // keys (0 = not selectable)
  uint32_t key[SEL_PER];
  if (MODE == 0) {
    const float* row = scores + q * ncols + start;
#pragma unroll
    for (int u = 0; u < SEL_PER; ++u) key[u] = pw + 64 * u < n ? select_key(row[pw + 64 * u]) : 0u;
  } else if (MODE == 2) {
    const float* row = scores + q * ncols;
    const int32_t* map = col_blocks + q * nblk_map;
#pragma unroll
    for (int u = 0; u < SEL_PER; ++u) {
      const int pp = pw + 64 * u;
      key[u] = 0u;
      if (pp < n) {
        const int64_t pos = start + pp;
        const int32_t blk = map[pos >> 3];
        const int64_t e = 8 * (int64_t)blk + (pos & 7);
        if (blk >= 0 && e < ncols) key[u] = select_key(row[e]);
      }
    }
  } else {
    const uint32_t* row = cand_keys + q * n_in + start;
#pragma unroll
    for (int u = 0; u < SEL_PER; ++u) key[u] = pw + 64 * u < n ? row[pw + 64 * u] : 0u;
  }

  // 1. largest / smallest valid key and the valid count
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu, nval = 0;
#pragma unroll
  for (int u = 0; u < SEL_PER; ++u) {
    kmax = key[u] > kmax ? key[u] : kmax;
    kmin = (key[u] != 0 && key[u] < kmin) ? key[u] : kmin;
    nval += key[u] != 0;
  }
  kmax = wave_reduce<0>(kmax);
  kmin = wave_reduce<1>(kmin);
  nval = wave_reduce<2>(nval);
  for (int b = tid; b < SEL_BINS; b += SEL_THREADS) s.hist[b] = 0;
  if (lane == 0) {
    s.wred[0][wv] = kmax;
    s.wred[1][wv] = kmin;
    s.wred[2][wv] = nval;
  }
  if (tid == 0) s.n_cand = 0;
  __syncthreads();
  kmax = 0; kmin = 0xFFFFFFFFu; nval = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    kmax = s.wred[0][w] > kmax ? s.wred[0][w] : kmax;
    kmin = s.wred[1][w] < kmin ? s.wred[1][w] : kmin;
    nval += s.wred[2][w];
  }

  uint32_t T = 0, take_eq = 0;     // T = 0: every valid key is taken
  if (nval > (uint32_t)K) {
    // 2. value-linear histogram and the bin of the K-th largest key
    const float vmax = key_value(kmax), vmin = key_value(kmin);
    const float range = vmax - vmin;
    const float inv = (range > 0.0f && range < __builtin_huge_valf()) ? (float)SEL_BINS / range : 0.0f;
#pragma unroll
    for (int u = 0; u < SEL_PER; ++u)
      if (key[u] != 0) atomicAdd(&s.hist[value_bin(key_value(key[u]), vmax, inv)], 1u);
    __syncthreads();
    const uint32_t h0 = s.hist[2 * tid], h1 = s.hist[2 * tid + 1];
    uint32_t tot;
    const uint32_t excl = block_excl_scan(s, h0 + h1, &tot);
    if (excl < (uint32_t)K && (uint32_t)K <= excl + h0 + h1) {
      const bool first = (uint32_t)K <= excl + h0;
      s.bstar = first ? 2 * tid : 2 * tid + 1;
      s.rem = first ? K - excl : K - excl - h0;
    }
    __syncthreads();
    const int bstar = (int)s.bstar;
    const uint32_t rem = s.rem;
    // 3. the exact K-th largest among the threshold bin's keys
#pragma unroll
    for (int u = 0; u < SEL_PER; ++u) {
      if (key[u] != 0 && value_bin(key_value(key[u]), vmax, inv) == bstar) {
        const uint32_t slot = atomicAdd(&s.n_cand, 1u);
        s.cand[slot] = key[u];
      }
    }
    __syncthreads();
    const int nc = (int)s.n_cand;
    if (nc <= SEL_RANK_MAX) {
      if (tid < nc) {
        const uint32_t ki = s.cand[tid];
        uint32_t g = 0, e = 0;
        for (int j = 0; j < nc; ++j) {
          const uint32_t kj = s.cand[j];
          g += kj > ki;
          e += kj == ki;
        }
        if (g < rem && rem <= g + e) {   // equal keys write equal values
          s.T = ki;
          s.take_eq = rem - g;
        }
      }
    } else {
      radix_select_cand(s, nc, rem);
    }
    __syncthreads();
    T = s.T;
    take_eq = s.take_eq;
  }

  // 4. position-ordered compaction: per-wave counts of keys > T and == T
  //    (packed), a block scan over the waves, then ballots within the wave
  uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
  for (int u = 0; u < SEL_PER; ++u) {
    gt_w += __popcll(__ballot(key[u] > T));
    eq_w += __popcll(__ballot(T != 0 && key[u] == T));
  }
  if (lane == 0) s.wred[0][wv] = gt_w | (eq_w << 16);
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int v = 0; v < SEL_WAVES; ++v) {
    const uint32_t x = s.wred[0][v];
    before += v < wv ? x : 0u;
    tot += x;
  }
  const uint32_t gt_before = before & 0xFFFFu, eq_before = before >> 16;
  const uint32_t n_sel = (tot & 0xFFFFu) + ((tot >> 16) < take_eq ? (tot >> 16) : take_eq);
  uint32_t slot_base = gt_before + (eq_before < take_eq ? eq_before : take_eq);
  uint32_t eq_seen = eq_before;
#pragma unroll
  for (int u = 0; u < SEL_PER; ++u) {
    const bool is_gt = key[u] > T, is_eq = T != 0 && key[u] == T;
    const uint64_t eq_b = __ballot(is_eq);
    const uint32_t eq_rank = eq_seen + __builtin_amdgcn_mbcnt_hi((uint32_t)(eq_b >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)eq_b, 0u));
    const bool take = is_gt || (is_eq && eq_rank < take_eq);
    const uint64_t tk_b = __ballot(take);
    const uint32_t slot = slot_base + __builtin_amdgcn_mbcnt_hi((uint32_t)(tk_b >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)tk_b, 0u));
    if (take && slot < (uint32_t)K) {
      const int pp = pw + 64 * u;
      int64_t col;
      if (MODE == 0) col = start + pp;
      else if (MODE == 1) col = cand_cols[q * n_in + start + pp];
      else col = 8 * (int64_t)col_blocks[q * nblk_map + ((start + pp) >> 3)] + ((start + pp) & 7);
      if (FINAL) {
        int64_t id = col;
        if (MODE == 0 && col_blocks) id = 8 * (int64_t)col_blocks[q * nblk_map + (col >> 3)] + (col & 7);
        idx[q * K + slot] = (int32_t)id;
      } else {
        const int64_t o = (q * gridDim.x + blockIdx.x) * (int64_t)K + slot;
        out_keys[o] = key[u];
        out_cols[o] = (int32_t)col;
      }
    }
    slot_base += (uint32_t)__popcll(tk_b);
    eq_seen += (uint32_t)__popcll(eq_b);
  }
  for (int j = (int)n_sel + tid; j < K; j += SEL_THREADS) {
    if (FINAL) {
      idx[q * K + j] = -1;
    } else {
      const int64_t o = (q * gridDim.x + blockIdx.x) * (int64_t)K + j;
      out_keys[o] = 0u;
      out_cols[o] = -1;
    }
  }
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
int64_t chunks_of(int64_t n) { return (n + SEL_CHUNK - 1) / SEL_CHUNK; }

// Candidate-buffer length per row needed by the multi-stage selection.
int64_t cand_len(int64_t ncols, int32_t k) {
  int64_t c = chunks_of(ncols);
  if (c <= 1) return 0;
  return c * (int64_t)k;
}
}  // namespace

size_t topk_workspace_bytes(int64_t Q, int64_t ncols, int32_t k) {
  int64_t len = cand_len(ncols, k);
  // two ping-pong candidate buffers of (key, column) pairs
  return (size_t)(2 * Q * len) * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_topk(const float* scores, int64_t Q, int64_t ncols, const int32_t* col_blocks,
                       int32_t k, int32_t* idx, void* ws, hipStream_t st) {
  if (Q == 0) return hipSuccess;
  int64_t nblk_map = (ncols + 7) >> 3;
  int64_t c = chunks_of(ncols);
  if (c <= 1) {
    hipLaunchKernelGGL((select_kernel<0, true>), dim3(1, (unsigned)Q), dim3(SEL_THREADS), 0, st, scores,
                       ncols, nullptr, nullptr, 0, col_blocks, nblk_map, k, idx, nullptr, nullptr);
    return hipGetLastError();
  }
  int64_t len = cand_len(ncols, k);
  uint32_t* keys0 = reinterpret_cast<uint32_t*>(ws);
  int32_t* cols0 = reinterpret_cast<int32_t*>(keys0 + Q * len);
  uint32_t* keys1 = reinterpret_cast<uint32_t*>(cols0 + Q * len);
  int32_t* cols1 = reinterpret_cast<int32_t*>(keys1 + Q * len);
  hipLaunchKernelGGL((select_kernel<0, false>), dim3((unsigned)c, (unsigned)Q), dim3(SEL_THREADS), 0, st,
                     scores, ncols, nullptr, nullptr, 0, nullptr, 0, k, nullptr, keys0, cols0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t n_in = c * k;
  while (chunks_of(n_in) > 1) {
    int64_t c2 = chunks_of(n_in);
    hipLaunchKernelGGL((select_kernel<1, false>), dim3((unsigned)c2, (unsigned)Q), dim3(SEL_THREADS), 0,
                       st, nullptr, 0, keys0, cols0, n_in, nullptr, 0, k, nullptr, keys1, cols1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint32_t* tk = keys0; keys0 = keys1; keys1 = tk;
    int32_t* tc = cols0; cols0 = cols1; cols1 = tc;
    n_in = c2 * k;
  }
  hipLaunchKernelGGL((select_kernel<1, true>), dim3(1, (unsigned)Q), dim3(SEL_THREADS), 0, st, nullptr, 0,
                     keys0, cols0, n_in, col_blocks, nblk_map, k, idx, nullptr, nullptr);
  return hipGetLastError();
}

size_t topk_gather_workspace_bytes(int64_t Q, int64_t nmap, int32_t k) {
  return topk_workspace_bytes(Q, 8 * nmap, k);
}

// K best entries among the entries of the listed blocks (MODE 2), ascending ids.
hipError_t launch_topk_gather(const float* scores, int64_t Q, int64_t ncols, const int32_t* blocks,
                              int64_t nmap, int32_t k, int32_t* idx, void* ws, hipStream_t st) {
  if (Q == 0) return hipSuccess;
  const int64_t n = 8 * nmap;
  int64_t c = chunks_of(n);
  if (c <= 1) {
    hipLaunchKernelGGL((select_kernel<2, true>), dim3(1, (unsigned)Q), dim3(SEL_THREADS), 0, st, scores,
                       ncols, nullptr, nullptr, n, blocks, nmap, k, idx, nullptr, nullptr);
    return hipGetLastError();
  }
  int64_t len = cand_len(n, k);
  uint32_t* keys0 = reinterpret_cast<uint32_t*>(ws);
  int32_t* cols0 = reinterpret_cast<int32_t*>(keys0 + Q * len);
  uint32_t* keys1 = reinterpret_cast<uint32_t*>(cols0 + Q * len);
  int32_t* cols1 = reinterpret_cast<int32_t*>(keys1 + Q * len);
  hipLaunchKernelGGL((select_kernel<2, false>), dim3((unsigned)c, (unsigned)Q), dim3(SEL_THREADS), 0, st,
                     scores, ncols, nullptr, nullptr, n, blocks, nmap, k, nullptr, keys0, cols0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t n_in = c * k;
  while (chunks_of(n_in) > 1) {
    int64_t c2 = chunks_of(n_in);
    hipLaunchKernelGGL((select_kernel<1, false>), dim3((unsigned)c2, (unsigned)Q), dim3(SEL_THREADS), 0,
                       st, nullptr, 0, keys0, cols0, n_in, nullptr, 0, k, nullptr, keys1, cols1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint32_t* tk = keys0; keys0 = keys1; keys1 = tk;
    int32_t* tc = cols0; cols0 = cols1; cols1 = tc;
    n_in = c2 * k;
  }
  hipLaunchKernelGGL((select_kernel<1, true>), dim3(1, (unsigned)Q), dim3(SEL_THREADS), 0, st, nullptr, 0,
                     keys0, cols0, n_in, nullptr, 0, k, idx, nullptr, nullptr);
  return hipGetLastError();
}

size_t block_pool_workspace_bytes(int64_t Q, int64_t ncols, int32_t is_block_max, int32_t nb) {
  int64_t nblk = is_block_max ? ncols : (ncols + 7) / 8;
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
    int64_t tot = Q * nblk;
    hipLaunchKernelGGL(block_max_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, values, Q,
                       ncols, tmp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bm = tmp;
    size_t used = ((size_t)tot * sizeof(float) + 255) & ~(size_t)255;
    rest += used;
  }
  return launch_topk(bm, Q, nblk, nullptr, nb, pool, rest, st);
}

}  // namespace csa

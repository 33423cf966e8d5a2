// Top-K selection and the hierarchical block pool.
//
// P3 §02: the first Full layer picks the Top-512 over every visible position,
// then ranks 8-position blocks by their largest score and keeps 2,048 of them
// (16,384 candidates) for the Reindex layers.  Equal scores go to the lower
// column (and so the lower entry id); -inf columns are never selected.
//
// Each block selects the K best of up to SEL_CHUNK keys held in LDS with an
// exact radix select (four 8-bit digit passes find the K-th largest key T and
// how many keys equal to T are still needed), then compacts the chosen
// positions in position order with wave ballots, which keeps the output
// ascending and resolves ties toward the lower position.  Rows longer than
// SEL_CHUNK are cut into chunks; every chunk's K best are kept as candidates
// (the global K best are among them) and selected again.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int SEL_CHUNK = 16384;
constexpr int SEL_THREADS = 512;
constexpr int SEL_WAVES = SEL_THREADS / 64;

namespace {

struct SelShared {
  uint32_t keys[SEL_CHUNK];
  uint32_t hist[256];
  uint32_t wave_cnt[SEL_WAVES];
  uint32_t wave_tot[4];
  uint32_t digit, remaining;
  uint32_t run_eq, run_sel;
};

// Block-wide exclusive prefix count of `flag`; returns the lane's rank and
// writes the block total to *total.  Uses s.wave_cnt; two barriers.
__device__ __forceinline__ uint32_t block_rank(SelShared& s, bool flag, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t m = __ballot(flag);
  uint32_t below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s.wave_cnt[wave] = __popcll(m);
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    uint32_t c = s.wave_cnt[w];
    off += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + below;
}

// Find T = the K-th largest of keys[0..n) (n > K).  Returns T and sets
// *take_eq to how many keys equal to T are selected (the lowest positions).
__device__ uint32_t radix_select(SelShared& s, int n, uint32_t K, uint32_t* take_eq) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0;
  if (tid == 0) s.remaining = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += SEL_THREADS) s.hist[i] = 0;
    __syncthreads();
    const uint32_t rem = s.remaining;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < n; i += SEL_THREADS) {
      uint32_t k = s.keys[i];
      if ((k & hi_mask) == prefix) atomicAdd(&s.hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // inclusive suffix sums over the 256 digits (larger digit = larger key),
    // 64 digits per wave in waves 0..3
    uint32_t h = 0, incl = 0;
    if (wave < 4) {
      h = s.hist[64 * wave + lane];
      incl = h;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = __shfl_down(incl, off);
        if (lane + off < 64) incl += o;
      }
      if (lane == 0) s.wave_tot[wave] = incl;
    }
    __syncthreads();
    if (wave < 4) {
      for (int w = wave + 1; w < 4; ++w) incl += s.wave_tot[w];
      uint32_t excl = incl - h;
      if (h > 0 && excl < rem && rem <= incl) {
        s.digit = 64 * wave + lane;
        s.remaining = rem - excl;
      }
    }
    __syncthreads();
    prefix |= s.digit << shift;
  }
  *take_eq = s.remaining;
  return prefix;
}

}  // namespace

// MODE 0: keys come from float scores [Q, ncols] (column = position);
// MODE 1: keys / columns come from candidate arrays [Q, n_in].
// FINAL: write ids ascending to idx [Q, K]; otherwise write the chunk's K
// best (key, column) pairs ascending to cand_out [Q, gridDim.x * K].
template <int MODE, bool FINAL>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const float* __restrict__ scores, int64_t ncols, const uint32_t* __restrict__ cand_keys,
    const int32_t* __restrict__ cand_cols, int64_t n_in, const int32_t* __restrict__ col_blocks,
    int64_t nblk_map, int32_t K, int32_t* __restrict__ idx, uint32_t* __restrict__ out_keys,
    int32_t* __restrict__ out_cols) {
  __shared__ SelShared s;
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.y;
  const int64_t total = MODE == 0 ? ncols : n_in;
  const int64_t start = (int64_t)blockIdx.x * SEL_CHUNK;
  const int n = (int)((total - start) < SEL_CHUNK ? (total - start) : SEL_CHUNK);
  if (MODE == 0) {
    const float* row = scores + q * ncols + start;
    for (int i = tid; i < n; i += SEL_THREADS) s.keys[i] = select_key(row[i]);
  } else {
    const uint32_t* row = cand_keys + q * n_in + start;
    for (int i = tid; i < n; i += SEL_THREADS) s.keys[i] = row[i];
  }
  if (tid == 0) { s.run_eq = 0; s.run_sel = 0; }
  __syncthreads();
  uint32_t T = 0, take_eq = 0;
  if (n > K) T = radix_select(s, n, (uint32_t)K, &take_eq);
  if (T == 0) take_eq = 0;   // the K-th largest is an excluded key: take only valid keys
  uint32_t run_eq = 0, run_sel = 0;
  for (int base = 0; base < n; base += SEL_THREADS) {
    int i = base + tid;
    uint32_t key = i < n ? s.keys[i] : 0u;
    bool is_eq = (i < n) && T != 0 && key == T;
    uint32_t eq_tot, sel_tot;
    uint32_t eq_rank = run_eq + block_rank(s, is_eq, &eq_tot);
    bool sel = (i < n) && (key > T || (is_eq && eq_rank < take_eq));
    uint32_t slot = run_sel + block_rank(s, sel, &sel_tot);
    if (sel && slot < (uint32_t)K) {
      int64_t col;
      if (MODE == 0) col = start + i;
      else col = cand_cols[q * n_in + start + i];
      if (FINAL) {
        int64_t id = col;
        if (col_blocks) id = 8 * (int64_t)col_blocks[q * nblk_map + (col >> 3)] + (col & 7);
        idx[q * K + slot] = (int32_t)id;
      } else {
        int64_t o = (q * gridDim.x + blockIdx.x) * (int64_t)K + slot;
        out_keys[o] = key;
        out_cols[o] = (int32_t)col;
      }
    }
    run_eq += eq_tot;
    run_sel += sel_tot;
  }
  for (int j = (int)run_sel + tid; j < K; j += SEL_THREADS) {
    if (FINAL) {
      idx[q * K + j] = -1;
    } else {
      int64_t o = (q * gridDim.x + blockIdx.x) * (int64_t)K + j;
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

// Block-wide exact Top-K selection over keys held in registers (device
// routines shared by the selection kernels and the fused Full-layer kernel).
//
// "DeepSeek-V4.1 架构解析" §02: the Top-512 of the visible scores, ties to the lower position.
// The method is described in select.hip.
#pragma once

#include "common.h"

namespace csa {

constexpr int SEL_BINS = 2048;
constexpr int SEL_RANK_MAX = 256;                      // pairwise ranking up to this many keys
constexpr int SEL_MAX_WAVES = 16;
constexpr int64_t SEL_CHUNK_MAX = 32768;               // keys of one block
constexpr int SEL_POOL_MAX = 4096;                     // pool size of the fused kernel
constexpr int SEL_CAND_MAX = 4096;                     // candidates of the sampled path

namespace sel {

struct SelShared {
  uint32_t hist[SEL_BINS];
  uint32_t cand[SEL_RANK_MAX];
  uint32_t ckey[SEL_CAND_MAX];    // sampled path: candidates in position order
  uint16_t cpos[SEL_CAND_MAX];
  uint32_t wred[3][SEL_MAX_WAVES];
  uint32_t bstar, rem, n_cand, T, take_eq, tlo;
};

// Key loads.  Every load below is issued unconditionally, from a clamped
// in-range address, and the bounds are applied to the loaded values: with a
// bound check around each load the compiler waits for every load in turn,
// which turns PER loads into PER round trips.
//
// key[u] = select_key(row[p]) for p = pw + 64 u < n, else 0 (n >= 0).
template <int PER>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int pw, int n, uint32_t (&key)[PER]) {
  if (n <= 0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) key[u] = 0u;
    return;
  }
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = pw + 64 * u;
    v[u] = row[p < n ? p : n - 1];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) key[u] = (pw + 64 * u < n) ? select_key(v[u]) : 0u;
}

// key[u] = row[p] (already a key) for p = pw + 64 u < n, else 0.
template <int PER>
__device__ __forceinline__ void load_raw_keys(const uint32_t* __restrict__ row, int pw, int n, uint32_t (&key)[PER]) {
  if (n <= 0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) key[u] = 0u;
    return;
  }
  uint32_t v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = pw + 64 * u;
    v[u] = row[p < n ? p : n - 1];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) key[u] = (pw + 64 * u < n) ? v[u] : 0u;
}

// Pooled positions: position p = pw + 64 u (< n) is entry 8 b + (p & 7) of
// row with b = block_of(p >> 3) (b < 0: no block); entries >= ncols are not
// selectable.  block_of is called for in-range block slots only.
template <int PER, class BlockOf>
__device__ __forceinline__ void gather_keys(const float* __restrict__ row, int64_t ncols, int pw, int n,
                                            BlockOf block_of, uint32_t (&key)[PER]) {
  if (n <= 0 || ncols <= 0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) key[u] = 0u;
    return;
  }
  int64_t e[PER];
  bool ok[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = pw + 64 * u;
    const int pc = p < n ? p : 0;
    const int32_t b = block_of(pc >> 3);
    const int64_t ee = 8 * (int64_t)b + (pc & 7);
    ok[u] = p < n && b >= 0 && ee < ncols;
    e[u] = ok[u] ? ee : 0;
  }
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) v[u] = row[e[u]];
#pragma unroll
  for (int u = 0; u < PER; ++u) key[u] = ok[u] ? select_key(v[u]) : 0u;
}

// Value of a valid (non-zero) key: the inverse of select_key.
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Cross-lane steps on the DPP network (gfx9 controls: quad_perm, row_shr,
// row_mirror, row_half_mirror, row_bcast15, row_bcast31).  A lane whose row is
// outside the row mask, or whose source lane is outside its row, keeps `old`.
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

// Wave-wide max / min, returned uniformly (the full result lands in lane 63).
template <int OP>   // 0 max, 1 min
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return OP == 0 ? (a > b ? a : b) : (a < b ? a : b); };
  const uint32_t id = OP == 1 ? 0xFFFFFFFFu : 0u;
  v = f(v, dpp<DPP_XOR1>(id, v));
  v = f(v, dpp<DPP_XOR2>(id, v));
  v = f(v, dpp<DPP_ROW_HALF_MIRROR>(id, v));
  v = f(v, dpp<DPP_ROW_MIRROR>(id, v));
  v = f(v, dpp<DPP_BCAST15, 0xA>(id, v));
  v = f(v, dpp<DPP_BCAST31, 0xC>(id, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Cross-wave combination of one word per wave (arr[0 .. W-1] in LDS, W <=
// 16): lane i < W of every wave reads arr[i] and the wave's first 16-lane row
// combines the words on the DPP network, so a thread reads one word instead
// of W and the sums take four steps instead of W.
// Sum over all waves; *before (if given) = the sum over waves below this one.
template <int W>
__device__ __forceinline__ uint32_t waves_sum(const uint32_t* arr, uint32_t* before) {
  static_assert(W >= 1 && W <= 16, "one DPP row");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = lane < W ? arr[lane] : 0u;
  x += dpp<DPP_ROW_SHR1>(0u, x);
  x += dpp<DPP_ROW_SHR2>(0u, x);
  x += dpp<DPP_ROW_SHR4>(0u, x);
  x += dpp<DPP_ROW_SHR8>(0u, x);   // lane i < 16: arr[0] + ... + arr[i]
  if (before) *before = wv == 0 ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)x, wv - 1);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, W - 1);
}
// Max (OP 0) or min (OP 1) over all waves.
template <int W, int OP>
__device__ __forceinline__ uint32_t waves_reduce(const uint32_t* arr) {
  static_assert(W >= 1 && W <= 16, "one DPP row");
  auto f = [](uint32_t a, uint32_t b) { return OP == 0 ? (a > b ? a : b) : (a < b ? a : b); };
  const uint32_t id = OP == 1 ? 0xFFFFFFFFu : 0u;
  const int lane = threadIdx.x & 63;
  uint32_t x = lane < W ? arr[lane] : id;
  x = f(x, dpp<DPP_XOR1>(id, x));
  x = f(x, dpp<DPP_XOR2>(id, x));
  x = f(x, dpp<DPP_ROW_HALF_MIRROR>(id, x));
  x = f(x, dpp<DPP_ROW_MIRROR>(id, x));   // every lane of row 0: the result
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
}

// Exclusive block scan of v; *total = the block sum.  One barrier: the
// caller passes another barrier before s.wred[0] is written again.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(SelShared& s, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) s.wred[0][wv] = incl;
  __syncthreads();
  uint32_t before;
  *total = waves_sum<NT / 64>(s.wred[0], &before);
  return before + incl - v;
}

// Bin of a valid value: 0 holds the largest values.
__device__ __forceinline__ int value_bin(uint32_t key, float vmax, float inv) {
  if (inv == 0.0f) return 0;
  const float x = (vmax - key_value(key)) * inv;
  return (int)fminf(x, (float)(SEL_BINS - 1));
}

// Thread t owns bins BPT t .. BPT t + BPT - 1 of h (already loaded): the bin
// where the running count from bin 0 reaches `need`, and how many of that
// bin's keys are needed.  Exactly one thread returns true.  Every caller
// passes a barrier before s.wred is written again (see block_excl_scan).
template <int NT, int BPT>
__device__ __forceinline__ bool find_bin(SelShared& s, const uint32_t (&h)[BPT], uint32_t need, int* bin,
                                         uint32_t* left) {
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) sum += h[j];
  uint32_t tot;
  const uint32_t excl = block_excl_scan<NT>(s, sum, &tot);
  if (!(excl < need && need <= excl + sum)) return false;
  uint32_t run = excl;
  bool found = false;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (!found && run + h[j] >= need) {
      *bin = BPT * (int)threadIdx.x + j;
      *left = need - run;
      found = true;
    }
    run += h[j];
  }
  return true;
}

template <int NT, int PER>
__device__ __forceinline__ void threshold_from_hist(SelShared& s, const uint32_t (&key)[PER], uint32_t K, float vmax,
                                                    float inv, uint32_t* T_out, uint32_t* take_out);

// Steps 1-3: the K-th largest key *T of the block's keys and how many keys
// equal to it are taken (*take_eq); T = 0 when at most K keys are valid (every
// valid key is taken).  Every thread of the block calls it.
template <int NT, int PER>
__device__ __forceinline__ void block_threshold(SelShared& s, const uint32_t (&key)[PER], uint32_t K,
                                                uint32_t* T_out, uint32_t* take_out) {
  constexpr int W = NT / 64, BPT = SEL_BINS / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu, nv_w = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    kmax = key[u] > kmax ? key[u] : kmax;
    kmin = (key[u] != 0 && key[u] < kmin) ? key[u] : kmin;
    nv_w += (uint32_t)__popcll(__ballot(key[u] != 0));
  }
  kmax = wave_reduce<0>(kmax);
  kmin = wave_reduce<1>(kmin);
  __syncthreads();   // earlier readers of the shared state are done
  for (int b = tid; b < SEL_BINS; b += NT) s.hist[b] = 0;
  if (lane == 0) {
    s.wred[0][wv] = kmax;
    s.wred[1][wv] = kmin;
    s.wred[2][wv] = nv_w;
  }
  if (tid == 0) s.n_cand = 0;
  __syncthreads();
  kmax = waves_reduce<W, 0>(s.wred[0]);
  kmin = waves_reduce<W, 1>(s.wred[1]);
  const uint32_t nval = waves_sum<W>(s.wred[2], nullptr);
  if (nval <= K) {
    *T_out = 0;
    *take_out = 0;
    return;
  }

  // 2. value-linear histogram and the bin of the K-th largest key
  const float vmax = key_value(kmax), vmin = key_value(kmin);
  const float range = vmax - vmin;
  const float inv = (range > 0.0f && range < __builtin_huge_valf()) ? (float)SEL_BINS / range : 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (key[u] != 0) atomicAdd(&s.hist[value_bin(key[u], vmax, inv)], 1u);
  __syncthreads();
  threshold_from_hist<NT, PER>(s, key, K, vmax, inv, T_out, take_out);
}

// Steps 2-3 once the value histogram of the valid keys (value_bin with vmax,
// inv; at least K of them) is in hist and s.n_cand is 0: the bin of the K-th
// largest key, then that key T exactly among the bin's keys (pairwise
// ranking when the bin holds at most SEL_RANK_MAX keys, else a radix select)
// and how many keys equal to T are taken.
template <int NT, int PER>
__device__ __forceinline__ void threshold_from_hist(SelShared& s, const uint32_t (&key)[PER], uint32_t K, float vmax,
                                                    float inv, uint32_t* T_out, uint32_t* take_out) {
  constexpr int BPT = SEL_BINS / NT;
  const int tid = threadIdx.x;
  {
    uint32_t h[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) h[j] = s.hist[BPT * tid + j];
    int bin;
    uint32_t left;
    if (find_bin<NT, BPT>(s, h, K, &bin, &left)) {
      s.bstar = (uint32_t)bin;
      s.rem = left;
    }
  }
  __syncthreads();
  const int bstar = (int)s.bstar;
  uint32_t rem = s.rem;
  const uint32_t nc = s.hist[bstar];
  uint64_t inbin = 0;   // bit u: key[u] lies in the threshold bin
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (key[u] != 0 && value_bin(key[u], vmax, inv) == bstar) inbin |= 1ull << u;

  // 3. the exact rem-th largest key of the threshold bin
  if (nc <= SEL_RANK_MAX) {
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if ((inbin >> u) & 1u) s.cand[atomicAdd(&s.n_cand, 1u)] = key[u];
    __syncthreads();
    for (int i = tid; i < (int)nc; i += NT) {
      const uint32_t ki = s.cand[i];
      uint32_t g = 0, e = 0;
      for (int j = 0; j < (int)nc; ++j) {
        const uint32_t kj = s.cand[j];
        g += kj > ki;
        e += kj == ki;
      }
      if (g < rem && rem <= g + e) {   // keys equal to ki write equal values
        s.T = ki;
        s.take_eq = rem - g;
      }
    }
    __syncthreads();
    *T_out = s.T;
    *take_out = s.take_eq;
    return;
  }
  uint32_t prefix = 0;
  const int shifts[3] = {21, 10, 0};
  const uint32_t masks[3] = {0u, 0xFFE00000u, 0xFFFFFC00u};
  for (int pass = 0; pass < 3; ++pass) {
    __syncthreads();   // earlier readers of hist / T / rem are done
    for (int b = tid; b < SEL_BINS; b += NT) s.hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (((inbin >> u) & 1u) && (key[u] & masks[pass]) == prefix)
        atomicAdd(&s.hist[(key[u] >> shifts[pass]) & (SEL_BINS - 1)], 1u);
    __syncthreads();
    // thread t owns digits 2047 - BPT t - j (largest digits first)
    uint32_t h[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) h[j] = s.hist[SEL_BINS - 1 - (BPT * tid + j)];
    int bin;
    uint32_t left;
    if (find_bin<NT, BPT>(s, h, rem, &bin, &left)) {
      s.T = (uint32_t)(SEL_BINS - 1 - bin);
      s.rem = left;
    }
    __syncthreads();
    prefix |= s.T << shifts[pass];
    rem = s.rem;
  }
  *T_out = prefix;
  *take_out = rem;
}

// Step 4: the selected keys (key > T, or key == T among the first take_eq in
// position order) get consecutive slots in position order; emit(u, slot) is
// called for every selected key with slot < K.  Returns the number selected.
template <int NT, int PER, class Emit>
__device__ __forceinline__ uint32_t block_compact(SelShared& s, const uint32_t (&key)[PER], uint32_t T,
                                                  uint32_t take_eq, uint32_t K, Emit emit) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    gt_w += (uint32_t)__popcll(__ballot(key[u] > T));
    eq_w += (uint32_t)__popcll(__ballot(T != 0 && key[u] == T));
  }
  __syncthreads();   // earlier readers of wred are done
  if (lane == 0) {
    s.wred[0][wv] = gt_w;
    s.wred[1][wv] = eq_w;
  }
  __syncthreads();
  uint32_t gt_before, eq_before;
  const uint32_t gt_tot = waves_sum<W>(s.wred[0], &gt_before);
  const uint32_t eq_tot = waves_sum<W>(s.wred[1], &eq_before);
  uint32_t slot_base = gt_before + (eq_before < take_eq ? eq_before : take_eq);
  uint32_t eq_seen = eq_before;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bool is_gt = key[u] > T, is_eq = T != 0 && key[u] == T;
    const uint64_t eq_b = __ballot(is_eq);
    const bool take = is_gt || (is_eq && eq_seen + lanes_below(eq_b) < take_eq);
    const uint64_t tk_b = __ballot(take);
    const uint32_t slot = slot_base + lanes_below(tk_b);
    if (take && slot < K) emit(u, slot);
    slot_base += (uint32_t)__popcll(tk_b);
    eq_seen += (uint32_t)__popcll(eq_b);
  }
  return gt_tot + (eq_tot < take_eq ? eq_tot : take_eq);
}

// Steps 2-4 over the n >= K candidates gathered in LDS (ckey / cpos,
// position order), CP per thread, whose values lie in [vlo, vmax] (hist is
// clear and s.n_cand is 0); emit(p, key, slot) with p from cpos.
template <int NT, int CP, class Emit>
__device__ __forceinline__ uint32_t select_candidates(SelShared& s, uint32_t n, uint32_t K, float vmax, float vlo,
                                                      Emit emit) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t ck[CP];
#pragma unroll
  for (int i = 0; i < CP; ++i) {
    const uint32_t c = 64 * CP * wv + 64 * i + lane;
    ck[i] = c < n ? s.ckey[c] : 0u;
  }
  const float range = vmax - vlo;
  const float inv = (range > 0.0f && range < __builtin_huge_valf()) ? (float)SEL_BINS / range : 0.0f;
#pragma unroll
  for (int i = 0; i < CP; ++i)
    if (ck[i] != 0) atomicAdd(&s.hist[value_bin(ck[i], vmax, inv)], 1u);
  __syncthreads();
  uint32_t T, take_eq;
  threshold_from_hist<NT, CP>(s, ck, K, vmax, inv, &T, &take_eq);
  return block_compact<NT, CP>(s, ck, T, take_eq, K, [&](int i, uint32_t slot) {
    const uint32_t c = 64 * CP * wv + 64 * i + lane;
    emit((int)s.cpos[c], ck[i], slot);
  });
}

// The K best keys of the block (thread layout as above; p = 64 PER v + 64 u + l
// is the position of key[u]): emit(p, key, slot) for each, slots ascending
// with p.  Returns the number selected (min(K, valid keys)).
//
// With 8+ keys per thread the K-th largest key is first bounded from below
// with a sample (one key per thread, spread over each wave's run): T_lo is
// the lower edge of the sample-histogram bin (between the smallest sample
// and the largest key) where the sample count reaches m, about
// 1.5 K n_sample / n (+8).  If the keys >= T_lo number between K and
// SEL_CAND_MAX, they hold the K best (every other key is smaller), so they
// are gathered in position order and selected exactly, their histogram
// spanning [T_lo, largest key]; otherwise the exact selection runs over all
// keys.
template <int NT, int PER, class Emit>
__device__ __forceinline__ uint32_t block_select(SelShared& s, const uint32_t (&key)[PER], uint32_t K, Emit emit) {
  constexpr int W = NT / 64, BPT = SEL_BINS / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int pw = 64 * PER * wv + lane;
  if constexpr (PER >= 8) {
    uint32_t nv_w = 0, smp = 0, kmx = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      nv_w += (uint32_t)__popcll(__ballot(key[u] != 0));
      smp = (u == lane % PER) ? key[u] : smp;
      kmx = key[u] > kmx ? key[u] : kmx;
    }
    kmx = wave_reduce<0>(kmx);
    const uint32_t smin = wave_reduce<1>(smp != 0 ? smp : 0xFFFFFFFFu);
    const uint32_t sv_w = (uint32_t)__popcll(__ballot(smp != 0));
    __syncthreads();   // earlier readers of the shared state are done
    for (int b = tid; b < SEL_BINS; b += NT) s.hist[b] = 0;
    if (lane == 0) {
      s.wred[0][wv] = kmx;
      s.wred[1][wv] = smin;
      s.wred[2][wv] = nv_w | (sv_w << 16);   // <= 32768 keys, <= 1024 samples
    }
    __syncthreads();
    const uint32_t kmax = waves_reduce<W, 0>(s.wred[0]), kmin = waves_reduce<W, 1>(s.wred[1]);
    const uint32_t packed = waves_sum<W>(s.wred[2], nullptr);   // sum of the 16-bit fields: no carry
    const uint32_t nval = packed & 0xFFFFu, sval = packed >> 16;
    const uint32_t m = (uint32_t)(1.5f * (float)K * (float)sval / (float)(nval > 0 ? nval : 1)) + 8u;
    if (nval > K && m < sval) {
      const float vmax = key_value(kmax), vmin = key_value(kmin);
      const float range = vmax - vmin;
      const float inv = (range > 0.0f && range < __builtin_huge_valf()) ? (float)SEL_BINS / range : 0.0f;
      if (smp != 0) atomicAdd(&s.hist[value_bin(smp, vmax, inv)], 1u);
      __syncthreads();
      {
        uint32_t h[BPT];
#pragma unroll
        for (int j = 0; j < BPT; ++j) h[j] = s.hist[BPT * tid + j];
        int bin;
        uint32_t left;
        if (find_bin<NT, BPT>(s, h, m, &bin, &left)) {
          uint32_t t = kmin;
          if (inv != 0.0f) {
            const float e = vmax - (float)(bin + 1) / inv;   // the bin's lower edge
            if (e > vmin) t = select_key(e);
          }
          s.tlo = t;
        }
      }
      __syncthreads();
      const uint32_t tlo = s.tlo;
      uint32_t c_w = 0;
#pragma unroll
      for (int u = 0; u < PER; ++u) c_w += (uint32_t)__popcll(__ballot(key[u] >= tlo));
      if (lane == 0) s.wred[0][wv] = c_w;
      for (int b = tid; b < SEL_BINS; b += NT) s.hist[b] = 0;   // for the candidates' histogram
      if (tid == 0) s.n_cand = 0;
      __syncthreads();
      uint32_t off;
      const uint32_t C = waves_sum<W>(s.wred[0], &off);
      if (C >= K && C <= SEL_CAND_MAX) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const bool in = key[u] >= tlo;
          const uint64_t mk = __ballot(in);
          if (in) {
            const uint32_t c = off + lanes_below(mk);
            s.ckey[c] = key[u];
            s.cpos[c] = (uint16_t)(pw + 64 * u);
          }
          off += (uint32_t)__popcll(mk);
        }
        __syncthreads();
        const float vlo = key_value(tlo);
        if (C <= 4 * NT) return select_candidates<NT, 4>(s, C, K, vmax, vlo, emit);
        return select_candidates<NT, SEL_CAND_MAX / NT>(s, C, K, vmax, vlo, emit);
      }
    }
  }
  uint32_t T, take_eq;
  block_threshold<NT, PER>(s, key, K, &T, &take_eq);
  return block_compact<NT, PER>(s, key, T, take_eq, K, [&](int u, uint32_t slot) { emit(pw + 64 * u, key[u], slot); });
}

}  // namespace sel

}  // namespace csa

// Sparse multi-query attention over the selected MXFP4 entries plus the
// FP8 sliding window.
//
// P3 §02: the selected Top-K entries are used for attention; one shared latent
// serves all query heads (fewer KV heads).  P3 §03: the FP4 cache is
// dequantized before attention (no FP4 matmul), the SWA window stays FP8 and
// covers n_win = 128 tokens.
//
// Work item = (query, split of its key slots); one block of KG key groups of
// four waves per work item, wave w of a group owning channels 128 w .. 128 w
// + 127, and group kg taking the split's tiles kg, kg + KG, ...  Key slots
// 0..k-1 are the selected entries, slots k..k+127 the window tokens
// p-127..p.  Per 16-slot tile:
//   1. lane (j, g) of wave w loads channels 128 w + 32 g .. + 31 of key j
//      (16 FP4 code bytes + 2 E4M3 scale bytes, or 32 E4M3 window bytes) and
//      dequantizes them to fp16 in registers (exact);
//   2. partial S^T = K Q^T over the wave's channels on the fp16 matrix cores
//      (4 x v_mfma 16x16x32), summed over the four waves through LDS in a
//      fixed order, so every wave holds the same S;
//   3. online softmax in float32 (log2 domain), computed alike by each wave;
//   4. the fp16 key slices go through the wave's own LDS rows so that each
//      lane can gather 4 keys of one channel for the B operand of P V
//      (8 x v_mfma 16x16x16).  Output channel of N-tile n in lane column c is
//      128 w + 8 c + n, so every lane reads 16 contiguous bytes per key.
// Key bytes are loaded at_depth tiles ahead of use and slot ids 2 at_depth
// tiles ahead.  The key groups of a block merge their (O, max, sum) through
// LDS at the end, so a split writes one partial however many groups it has;
// with several splits per query the partials are combined by
// attn_combine_kernel.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int AT_TILE = 16;
constexpr int AT_WAVES = 4;                      // waves of one key group
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_QCH = D / AT_WAVES;             // channels per wave
constexpr int AT_KPITCH = AT_QCH * 2 + 16;       // bytes per LDS key row of one wave (fp16 + pad)
// Tiles of key bytes in flight: two with several key groups per block (few
// blocks, so the loads' latency shows), one with a single group (four
// waves per SIMD, whose interleaving covers the latency of one tile ahead;
// one register set fewer to rotate).
template <int KG> constexpr int at_depth() { return KG == 1 ? 1 : 2; }

struct AttnArgs {
  const float* q;
  const int32_t* q_pos;
  int64_t q_per_seq;
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t kv_rows;
  const int32_t* idx;
  int32_t k;
  const uint8_t* win;
  int64_t win_cap;
  float c_log2;          // sm_scale * log2(e)
  float* out;
  float* part_o;         // [Q, n_splits, 16, 512] (n_splits > 1)
  float* part_ml;        // [Q, n_splits, 2, 16]
  int n_splits;
  int tiles_per_split;
};

// One lane's 32 channels of one key: entry = 16 FP4 code bytes (a) and the
// two E4M3 scales of its 16-channel groups (sc); window = 32 E4M3 bytes
// (a, b).  kind: 0 = no key (all bytes zero, so it dequantizes to 0),
// 1 = entry, 2 = window token.
struct RawKey {
  uint4 a, b;
  uint32_t sc;
  int32_t kind;
};

// Tile kinds, wave-uniform: all slots selected entries, all window slots, or
// both (only when k is not a multiple of the tile, in the one tile holding
// slot k).  Padding slots are kind 0 and fit every tile kind.
constexpr int TK_ENTRY = 0, TK_WINDOW = 1, TK_MIXED = 2;
// Kind of tile t (t * AT_TILE is the same in every lane).
__device__ __forceinline__ int tile_kind(int t, int k) {
  const int slot0 = t * AT_TILE;
  return slot0 + AT_TILE <= k ? TK_ENTRY : slot0 >= k ? TK_WINDOW : TK_MIXED;
}

// Entry id of this lane's slot in tile t (-1: padding / out of range; the
// window slots need no id).  idx_q is the query's row of the index array.
__device__ __forceinline__ int32_t slot_id(const int32_t* idx_q, int k, int t, int t_end, int j) {
  const int slot = t * AT_TILE + j;
  if (t >= t_end || slot >= k) return -1;
  return idx_q[slot];
}

// wbase is the ring row of position p - 127 (mod win_cap, win_cap >= 128),
// so window slot wi sits at row wbase + wi, wrapped at most once.
// TK (see below) is the kind of tile t, the same for every lane: an entry
// tile loads no window bytes and a window tile no entry bytes.
template <int TK>
__device__ __forceinline__ RawKey load_key(const AttnArgs& a, int t, int t_end, int j, int g, int w,
                                           int32_t id, int32_t p, int64_t wbase, const uint8_t* codes_seq,
                                           const uint8_t* scales_seq, const uint8_t* win_seq) {
  RawKey r;
  r.a = make_uint4(0u, 0u, 0u, 0u);
  r.b = make_uint4(0u, 0u, 0u, 0u);
  r.sc = 0u;
  r.kind = 0;
  if (t >= t_end) return r;
  const int slot = t * AT_TILE + j;
  const bool entry_slot = (TK == TK_ENTRY) ? true : (TK == TK_WINDOW) ? false : slot < a.k;
  if (entry_slot) {
    if (id >= 0 && id < a.kv_rows) {
      r.a = *reinterpret_cast<const uint4*>(codes_seq + (int64_t)id * CODE_BYTES + 64 * w + 16 * g);
      r.sc = *reinterpret_cast<const uint16_t*>(scales_seq + (int64_t)id * SCALE_BYTES + 8 * w + 2 * g);
      r.kind = 1;
    }
  } else {
    const int wi = slot - a.k;
    if (wi < NWIN && p - (NWIN - 1) + wi >= 0) {
      int64_t row = wbase + wi;
      row = row >= a.win_cap ? row - a.win_cap : row;
      const uint4* src = reinterpret_cast<const uint4*>(win_seq + row * D + AT_QCH * w + 32 * g);
      r.a = src[0];
      r.b = src[1];
      r.kind = 2;
    }
  }
  return r;
}

// Channels 8 s .. 8 s + 7 of the lane's 32 as fp16 (exact), k-step s < 4.
// Window token: E4M3 bytes 8 s .. 8 s + 7.  Entry: code dword s (two
// channels per byte) times the scale of group s / 2.  A key of kind 0 has
// all bytes zero and gives +0 either way.
__device__ __forceinline__ f16x8 window_slice(const RawKey& r, int s) {
  const uint32_t wd[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
  const f16x2 a = fp8x2_to_f16<0>(wd[2 * s]), b = fp8x2_to_f16<1>(wd[2 * s]);
  const f16x2 c = fp8x2_to_f16<0>(wd[2 * s + 1]), d = fp8x2_to_f16<1>(wd[2 * s + 1]);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ f16x8 entry_slice(const RawKey& r, int s) {
  const uint32_t wd[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
  const f16x2 sc2 = fp8x2_to_f16<0>(r.sc);
  const _Float16 scale = (s < 2) ? sc2[0] : sc2[1];
  const f16x2 sp = f16x2{scale, scale};
  const uint32_t cw = wd[s];
  const f16x2 a = fp4x2_to_f16<0>(cw) * sp, b = fp4x2_to_f16<1>(cw) * sp;
  const f16x2 c = fp4x2_to_f16<2>(cw) * sp, d = fp4x2_to_f16<3>(cw) * sp;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
template <int TK>
__device__ __forceinline__ f16x8 key_slice(const RawKey& r, int s) {
  if constexpr (TK == TK_ENTRY) return entry_slice(r, s);
  else if constexpr (TK == TK_WINDOW) return window_slice(r, s);
  else return r.kind == 2 ? window_slice(r, s) : entry_slice(r, s);
}

// Rescale threshold of the online softmax (log2 units): the running reference
// max of a head moves only when a new logit exceeds it by more than this, so
// unnormalized weights stay <= 2^8 (exact range for fp16 P and fp32 sums)
// and O is rarely rescaled.
constexpr float AT_RESCALE = 8.0f;

// 2^x on the transcendental unit alone (v_exp_f32, ~1 ulp): the loop's
// arguments are <= AT_RESCALE or -inf (-> 0), and a weight that underflows to
// 0 is below anything the fp32 sums could hold, so the denormal range
// handling of exp2f is not needed there.
__device__ __forceinline__ float exp2_loop(float x) { return __builtin_amdgcn_exp2f(x); }

template <int KG>
struct AttnLds {
  union {
    struct {
      uint8_t k[KG * AT_WAVES][AT_TILE * AT_KPITCH];   // fp16 key slices, per wave
      f32x4 s[2][KG][AT_WAVES][64];                      // partial S, double-buffered by tile parity
    } loop;
    struct {
      float o[KG > 1 ? KG - 1 : 1][AT_WAVES][32][64];     // scaled O of groups 1..KG-1
      float ml[KG][2][HEADS];                            // (max, sum) per group and head
    } red;
  };
};

// Four waves per SIMD: registers capped at 128 per lane.
template <int KG>
__global__ __launch_bounds__(AT_THREADS * KG) __attribute__((amdgpu_waves_per_eu(4))) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnLds<KG> lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = (tid >> 6) & (AT_WAVES - 1);
  // the key group is wave-uniform: taken from lane 0, so the tile index and
  // every branch on it are scalar
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 8);
  constexpr int AT_DEPTH = at_depth<KG>();
  const int j = lane & 15;      // key slot (loads, S rows), head (Q, softmax), channel group (P V)
  const int g = lane >> 4;      // 32-channel group (loads), key group of 4 (S, P)
  const int64_t qi = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t seq = qi / a.q_per_seq;
  const int32_t p = a.q_pos[qi];
  const int n_slots = a.k + NWIN;
  const int n_tiles = (n_slots + AT_TILE - 1) / AT_TILE;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  t_end = t_end < n_tiles ? t_end : n_tiles;
  // group kg takes tiles t_begin + kg + KG i; every group runs n_iter rounds
  // (a round past t_end is all padding), so the block barriers line up
  const int n_iter = (t_end - t_begin + KG - 1) / KG;
  const uint8_t* codes_seq = a.codes + seq * a.kv_rows * CODE_BYTES;
  const uint8_t* scales_seq = a.scales + seq * a.kv_rows * SCALE_BYTES;
  const uint8_t* win_seq = a.win + seq * a.win_cap * D;
  auto tile = [&](int i) { return t_begin + kg + KG * i; };

  // Q: head j, channels 128 w + 32 g .. + 31 (issued first: nothing depends on it)
  float4 qraw[8];
  {
    const float4* src = reinterpret_cast<const float4*>(a.q + (qi * HEADS + j) * D + AT_QCH * w + 32 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) qraw[i] = src[i];
  }
  const int32_t* idx_q = a.idx + qi * a.k;
  int64_t wbase = ((int64_t)p - (NWIN - 1)) % a.win_cap;
  wbase = wbase < 0 ? wbase + a.win_cap : wbase;
  int32_t id_ahead[AT_DEPTH];
#pragma unroll
  for (int i = 0; i < AT_DEPTH; ++i) id_ahead[i] = slot_id(idx_q, a.k, tile(AT_DEPTH + i), t_end, j);
  RawKey ring[AT_DEPTH];
  // loads of tile t, dispatched on its kind (a scalar branch)
  auto issue = [&](int t, int32_t id) -> RawKey {
    const int tk = tile_kind(t, a.k);
    if (tk == TK_ENTRY) return load_key<TK_ENTRY>(a, t, t_end, j, g, w, id, p, wbase, codes_seq, scales_seq, win_seq);
    if (tk == TK_WINDOW) return load_key<TK_WINDOW>(a, t, t_end, j, g, w, id, p, wbase, codes_seq, scales_seq, win_seq);
    return load_key<TK_MIXED>(a, t, t_end, j, g, w, id, p, wbase, codes_seq, scales_seq, win_seq);
  };
#pragma unroll
  for (int i = 0; i < AT_DEPTH; ++i) ring[i] = issue(tile(i), slot_id(idx_q, a.k, tile(i), t_end, j));
  // Q carries the logit scale (sm_scale * log2 e), so S is already in the
  // log2 domain of the softmax
  f16x8 qf[4];
  const float cq = a.c_log2;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float4 x = qraw[2 * s], y = qraw[2 * s + 1];
    qf[s] = f16x8{(_Float16)(x.x * cq), (_Float16)(x.y * cq), (_Float16)(x.z * cq), (_Float16)(x.w * cq),
                  (_Float16)(y.x * cq), (_Float16)(y.y * cq), (_Float16)(y.z * cq), (_Float16)(y.w * cq)};
  }

  f32x4 acc_o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc_o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  uint8_t* krow = lds.loop.k[AT_WAVES * kg + w];

  for (int it = 0; it < n_iter; ++it) {
    const RawKey cur = ring[0];
#pragma unroll
    for (int i = 0; i + 1 < AT_DEPTH; ++i) ring[i] = ring[i + 1];
    ring[AT_DEPTH - 1] = issue(tile(it + AT_DEPTH), id_ahead[0]);
#pragma unroll
    for (int i = 0; i + 1 < AT_DEPTH; ++i) id_ahead[i] = id_ahead[i + 1];
    id_ahead[AT_DEPTH - 1] = slot_id(idx_q, a.k, tile(it + 2 * AT_DEPTH), t_end, j);

    // ---- 2. partial S^T over this wave's channels; slices to LDS row j ------
    __builtin_amdgcn_wave_barrier();   // the previous tile's LDS reads come first
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    auto qk = [&](auto tk) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 av = key_slice<decltype(tk)::value>(cur, s);
        *reinterpret_cast<f16x8*>(krow + j * AT_KPITCH + 64 * g + 16 * s) = av;
        sacc = mfma_f16_16x16x32(av, qf[s], sacc);
      }
    };
    // one conversion per tile kind
    const int tk = tile_kind(tile(it), a.k);
    if (tk == TK_ENTRY) qk(std::integral_constant<int, TK_ENTRY>{});
    else if (tk == TK_WINDOW) qk(std::integral_constant<int, TK_WINDOW>{});
    else qk(std::integral_constant<int, TK_MIXED>{});
    const int par = it & 1;
    lds.loop.s[par][kg][w][lane] = sacc;
    __syncthreads();
    f32x4 S = lds.loop.s[par][kg][0][lane];
#pragma unroll
    for (int v = 1; v < AT_WAVES; ++v) {
      const f32x4 o = lds.loop.s[par][kg][v][lane];
      S[0] += o[0]; S[1] += o[1]; S[2] += o[2]; S[3] += o[3];
    }

    // ---- 3. online softmax (lane: keys 4g+r, head j), lazy rescaling --------
    const uint32_t vmask = (uint32_t)(__ballot(cur.kind != 0) & 0xFFFFull);
    float x[4] = {S[0], S[1], S[2], S[3]};
    if (vmask != 0xFFFFu) {   // wave-uniform: only tiles with an absent key mask
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = ((vmask >> (4 * g + r)) & 1u) ? x[r] : -__builtin_huge_valf();
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max_xor32(max_xor16(mx));
    const bool first = (m_run == -__builtin_huge_valf());
    const bool move = !first && (mx > m_run + AT_RESCALE);
    if (__ballot(move)) {
      const float alpha = move ? exp2_loop(m_run - mx) : 1.0f;
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        acc_o[n][0] *= al[0]; acc_o[n][1] *= al[1];
        acc_o[n][2] *= al[2]; acc_o[n][3] *= al[3];
      }
    }
    if (first || move) m_run = mx;
    const float base = (m_run == -__builtin_huge_valf()) ? 0.f : m_run;
    float pr[4], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = exp2_loop(x[r] - base);
      psum += pr[r];
    }
    l_run += psum;   // this lane's keys only; the four lanes of head j are summed after the loop
    const f16x4 pa = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};

    // ---- 4. P V: gather keys 4g .. 4g+3 of channels 8j .. 8j+7 from LDS ---------
    uint4 v[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      v[kk] = *reinterpret_cast<const uint4*>(krow + (4 * g + kk) * AT_KPITCH + 16 * j);
    const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
    const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
    const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
    const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // channel pair (2i, 2i+1) of the 8: N-tiles 2i and 2i+1
      const f16x2 a0 = bits_f16x2(__builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u));
      const f16x2 a1 = bits_f16x2(__builtin_amdgcn_perm(w3[i], w2[i], 0x05040100u));
      const f16x2 b0 = bits_f16x2(__builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u));
      const f16x2 b1 = bits_f16x2(__builtin_amdgcn_perm(w3[i], w2[i], 0x07060302u));
      const f16x4 blo = {a0[0], a0[1], a1[0], a1[1]};
      const f16x4 bhi = {b0[0], b0[1], b1[0], b1[1]};
      acc_o[2 * i] = mfma_f16_16x16x16(pa, blo, acc_o[2 * i]);
      acc_o[2 * i + 1] = mfma_f16_16x16x16(pa, bhi, acc_o[2 * i + 1]);
    }
  }

  l_run = sum_xor32(sum_xor16(l_run));   // head j's sum over all keys of this group

  // ---- merge the key groups: O, max and sum per head over the groups --------
  // lane holds O[head 4g + r][channel 128 w + 8 j + n]; m_run, l_run are head j's
  float lsum[4];   // sum of head 4 g + r over the groups
  if constexpr (KG > 1) {
    __syncthreads();                                   // loop LDS is free
    if (w == 0 && lane < 16) {
      lds.red.ml[kg][0][j] = m_run;
      lds.red.ml[kg][1][j] = l_run;
    }
    __syncthreads();
    float mine[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      float M = lds.red.ml[0][0][h];
#pragma unroll
      for (int v = 1; v < KG; ++v) M = fmaxf(M, lds.red.ml[v][0][h]);
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < KG; ++v) {
        const float mv = lds.red.ml[v][0][h];
        const float sv = (mv == -__builtin_huge_valf()) ? 0.f : exp2f(mv - M);
        L = fmaf(sv, lds.red.ml[v][1][h], L);
        if (v == kg) mine[r] = sv;
      }
      lsum[r] = L;
    }
    // head j's merged max and sum (what a partial carries)
    {
      float M = lds.red.ml[0][0][j];
#pragma unroll
      for (int v = 1; v < KG; ++v) M = fmaxf(M, lds.red.ml[v][0][j]);
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < KG; ++v) {
        const float mv = lds.red.ml[v][0][j];
        L = fmaf((mv == -__builtin_huge_valf()) ? 0.f : exp2f(mv - M), lds.red.ml[v][1][j], L);
      }
      m_run = M;
      l_run = L;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      acc_o[n][0] *= mine[0]; acc_o[n][1] *= mine[1];
      acc_o[n][2] *= mine[2]; acc_o[n][3] *= mine[3];
    }
    if (kg > 0) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) lds.red.o[kg - 1][w][4 * n + r][lane] = acc_o[n][r];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int v = 0; v < KG - 1; ++v)
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_o[n][r] += lds.red.o[v][w][4 * n + r][lane];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = __shfl(l_run, 4 * g + r);
  }

  // ---- epilogue (group 0) ---------------------------------------------------
  if (a.n_splits == 1) {
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) inv[r] = lsum[r] > 0.f ? 1.0f / lsum[r] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(a.out + (qi * HEADS + 4 * g + r) * D + AT_QCH * w + 8 * j);
      dst[0] = make_float4(acc_o[0][r] * inv[r], acc_o[1][r] * inv[r], acc_o[2][r] * inv[r], acc_o[3][r] * inv[r]);
      dst[1] = make_float4(acc_o[4][r] * inv[r], acc_o[5][r] * inv[r], acc_o[6][r] * inv[r], acc_o[7][r] * inv[r]);
    }
  } else {
    const int64_t ps = qi * a.n_splits + split;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(a.part_o + (ps * HEADS + 4 * g + r) * D + AT_QCH * w + 8 * j);
      dst[0] = make_float4(acc_o[0][r], acc_o[1][r], acc_o[2][r], acc_o[3][r]);
      dst[1] = make_float4(acc_o[4][r], acc_o[5][r], acc_o[6][r], acc_o[7][r]);
    }
    if (w == 0 && lane < 16) {
      a.part_ml[(ps * 2 + 0) * HEADS + j] = m_run;
      a.part_ml[(ps * 2 + 1) * HEADS + j] = l_run;
    }
  }
}

// out[q, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.  One block of
// 128 threads per (query, head), 4 channels per thread; all split loads are
// issued before any use (the splits are independent).
constexpr int AT_MAX_SPLITS = 16;

__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, float* __restrict__ out) {
  const int64_t qi = blockIdx.y;
  const int h = blockIdx.x;
  float m[AT_MAX_SPLITS], l[AT_MAX_SPLITS];
  float4 o[AT_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < AT_MAX_SPLITS; ++s) {
    if (s < n_splits) {
      const int64_t ps = qi * n_splits + s;
      m[s] = part_ml[(ps * 2) * HEADS + h];
      l[s] = part_ml[(ps * 2 + 1) * HEADS + h];
      o[s] = reinterpret_cast<const float4*>(part_o + (ps * HEADS + h) * D)[threadIdx.x];
    }
  }
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < AT_MAX_SPLITS; ++s)
    if (s < n_splits) M = fmaxf(M, m[s]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < AT_MAX_SPLITS; ++s) {
    if (s < n_splits) {
      float wgt = (m[s] == -__builtin_huge_valf()) ? 0.f : exp2f(m[s] - M);
      L = fmaf(wgt, l[s], L);
      acc.x = fmaf(wgt, o[s].x, acc.x); acc.y = fmaf(wgt, o[s].y, acc.y);
      acc.z = fmaf(wgt, o[s].z, acc.z); acc.w = fmaf(wgt, o[s].w, acc.w);
    }
  }
  float inv = L > 0.f ? 1.0f / L : 0.f;
  reinterpret_cast<float4*>(out + (qi * HEADS + h) * D)[threadIdx.x] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

namespace {
struct AttnPlan {
  int kg, n_splits, tiles_per_split;
};

// Below 512 queries (decode batches) a query's slots go to 4 splits of two
// key groups each: the first tile's dependent gather (slot id, then the
// entry bytes) dominates a block's time, so each group takes several tiles,
// and four partials per query keep the combine small.  From 512 queries on,
// one group and one split per query (no partials).
AttnPlan attn_plan(int64_t Q, int32_t k) {
  const int n_tiles = (k + NWIN + AT_TILE - 1) / AT_TILE;
  int kg = 1, want = 1;
  if (Q < 512) {
    kg = 2;
    want = 4;
  }
  // at least KG tiles (one per group) per split
  int max_split = n_tiles / kg;
  max_split = max_split < 1 ? 1 : max_split;
  max_split = max_split < AT_MAX_SPLITS ? max_split : AT_MAX_SPLITS;
  int s = want < max_split ? want : max_split;
  s = s < 1 ? 1 : s;
  AttnPlan pl;
  pl.kg = kg;
  pl.tiles_per_split = (n_tiles + s - 1) / s;
  pl.n_splits = (n_tiles + pl.tiles_per_split - 1) / pl.tiles_per_split;
  return pl;
}
}  // namespace

size_t attn_workspace_bytes(int64_t Q, int32_t k) {
  const AttnPlan pl = attn_plan(Q, k);
  if (pl.n_splits <= 1) return 0;
  size_t po = (size_t)Q * pl.n_splits * HEADS * D * sizeof(float);
  size_t pm = (size_t)Q * pl.n_splits * 2 * HEADS * sizeof(float);
  return po + pm;
}

hipError_t launch_sparse_attn(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                              const uint8_t* codes, const uint8_t* scales, int64_t kv_rows,
                              const int32_t* idx, int32_t k, const uint8_t* win, int64_t win_cap,
                              float sm_scale, float* out, void* ws, hipStream_t st) {
  int64_t Q = n_seq * q_per_seq;
  if (Q == 0) return hipSuccess;
  AttnArgs a;
  a.q = q; a.q_pos = q_pos; a.q_per_seq = q_per_seq;
  a.codes = codes; a.scales = scales; a.kv_rows = kv_rows;
  a.idx = idx; a.k = k; a.win = win; a.win_cap = win_cap;
  a.c_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  const AttnPlan pl = attn_plan(Q, k);
  a.n_splits = pl.n_splits;
  a.tiles_per_split = pl.tiles_per_split;
  a.part_o = nullptr; a.part_ml = nullptr;
  if (a.n_splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)Q * a.n_splits * HEADS * D;
  }
  const dim3 grid(a.n_splits, (unsigned)Q);
  if (pl.kg == 2) hipLaunchKernelGGL(attn_kernel<2>, grid, dim3(AT_THREADS * 2), 0, st, a);
  else hipLaunchKernelGGL(attn_kernel<1>, grid, dim3(AT_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(HEADS, (unsigned)Q), dim3(128), 0, st, a.part_o, a.part_ml,
                     a.n_splits, out);
  return hipGetLastError();
}

}  // namespace csa

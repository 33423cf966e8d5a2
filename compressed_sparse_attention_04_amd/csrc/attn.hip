// Sparse multi-query attention over the selected MXFP4 entries plus the
// FP8 sliding window.
//
// "DeepSeek-V4.1 架构解析" §02 (CSA2): the selected Top-K entries are the
// keys of the attention, and one shared latent serves every query head (the
// number of KV heads is compressed).  §03 (精度与状态重建): the FP4 cache is
// dequantized before the attention (FP4 is a storage format, not a matmul
// format), and the sliding-window KV stays in FP8 over the last n_win = 128
// tokens.
//
// Key slots 0..k-1 of a query are its selected entries, slots k..k+127 the
// window tokens p-127..p.  A key group is four waves; wave w owns channels
// 128 w .. 128 w + 127.  Per 16-slot tile:
//   1. lane (j, g) of wave w holds channels 128 w + 32 g .. + 31 of slot j
//      (16 FP4 code bytes + 2 E4M3 scale bytes, or 32 E4M3 window bytes) and
//      widens them to fp16 in registers (exact: E2M1 x E4M3 needs 5
//      significant bits);
//   2. partial S^T = K Q^T over the wave's channels on the fp16 matrix cores.
//      Q is carried as two fp16 halves, hi = fp16(q) and lo = fp16(q - hi),
//      each contracted with the same exact keys (16x16x32, float32
//      accumulation), so S carries q to about 2^-22 instead of fp16's 2^-11;
//      the four waves' partials are summed through LDS in a fixed order, so
//      every wave holds the same S;
//   3. online softmax in float32 (log2 domain; every wave computes the same);
//   4. P V on the matrix cores with P split the same way: P_hi V + P_lo V
//      (16x16x16, exact products, float32 accumulation), so the weights
//      enter at ~2^-22 relative (the denominator sums the float32 weights,
//      which the two halves match to that order).  The fp16 key slices go
//      through the wave's own LDS rows,
//      and a transposed LDS read gives each lane 4 keys of one channel
//      (N-tile n, lane column c: channel 128 w + 16 n + c).
// Key bytes are read through buffer views of the query's rows: an absent
// key (a -1 id, an id past the cache, a window position before 0, padding)
// reads past the view and gets zeros, so no load sits under a branch: every
// slot issues its entry loads and its window loads, and the one that is not
// its kind returns zeros.
//
// Two launch shapes:
//   * pair (decode batches): a query's key slots are cut into splits of
//     four 32-slot pairs, each loaded whole before use, so the dependent
//     gather (slot id, then the entry bytes) is paid once per block; the P V
//     product contracts 32 keys per MFMA.  Splits write (O, max, sum)
//     partials that attn_combine_kernel merges.
//   * stream (prefill chunks, and decode with very large k): one block per
//     query (or a few splits), tiles streamed with one (one group) or two
//     (two groups) tiles of key bytes in flight.
// The key groups of a block merge their (O, max, sum) through LDS at the end.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int AT_TILE = 16;
constexpr int AT_WAVES = 4;                      // waves of one key group
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_QCH = D / AT_WAVES;             // channels per wave
constexpr int AT_KPITCH = AT_QCH * 2 + 16;       // bytes per LDS key row of one wave (fp16 + pad)
// Buffer offset past every view: the views hold fewer than 2^31 bytes
// (kv_rows <= 2^23 entries of 256 bytes, win_cap < 2^22 rows of 512 bytes).
constexpr uint32_t AT_OOB = 0x80000000u;

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
  int64_t n_queries;
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
__device__ __forceinline__ int tile_kind(int t, int k) {
  const int slot0 = t * AT_TILE;
  return slot0 + AT_TILE <= k ? TK_ENTRY : slot0 >= k ? TK_WINDOW : TK_MIXED;
}

// Buffer views of one query's rows and its window geometry.
struct QueryView {
  __amdgpu_buffer_rsrc_t codes, scales, win, idx;
  int32_t p;         // query position
  int32_t wbase;     // ring row of position p - 127 (mod win_cap)
  int32_t win_cap;
};

__device__ __forceinline__ QueryView query_view(const AttnArgs& a, int64_t qi) {
  const int64_t seq = qi / a.q_per_seq;
  QueryView v;
  v.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(a.codes + seq * a.kv_rows * CODE_BYTES), (short)0,
                                              (int)(a.kv_rows * CODE_BYTES), 0x00020000);
  v.scales = __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales + seq * a.kv_rows * SCALE_BYTES), (short)0,
                                               (int)(a.kv_rows * SCALE_BYTES), 0x00020000);
  v.win = __builtin_amdgcn_make_buffer_rsrc((void*)(a.win + seq * a.win_cap * D), (short)0, (int)(a.win_cap * D),
                                            0x00020000);
  v.idx = __builtin_amdgcn_make_buffer_rsrc((void*)(a.idx + qi * a.k), (short)0, a.k * 4, 0x00020000);
  v.p = a.q_pos[qi];
  v.win_cap = (int32_t)a.win_cap;
  int32_t wb = (int32_t)(((int64_t)v.p - (NWIN - 1)) % a.win_cap);
  v.wbase = wb < 0 ? wb + v.win_cap : wb;
  return v;
}

// The index-array word of this lane's slot j in tile t, loaded
// unconditionally: a slot that is not an entry slot (or a tile past the ones
// in use) reads past the index view and gets 0, which load_slot's own slot
// test discards.  (Applying that test here would put the result under a
// branch and make the compiler wait for the load on the spot.)
__device__ __forceinline__ int32_t slot_id(const QueryView& v, int k, int t, bool live, int j) {
  const int slot = t * AT_TILE + j;
  const uint32_t off = (live && slot < k) ? (uint32_t)slot * 4u : AT_OOB;
  return __builtin_amdgcn_raw_buffer_load_b32(v.idx, off, 0, 0);
}

__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
}

// The lane's bytes of slot j of tile t: the code and scale bytes of its
// entry and the bytes of its window token.  All four loads are issued in
// every lane (straight-line code: no register of a load in flight is copied
// at a branch join, and the compiler counts the loads in flight instead of
// waiting); a slot that is not an entry (or not a window token) reads past
// that view and gets zeros, so OR-ing the code and window bytes keeps
// whichever the slot is.
__device__ __forceinline__ uint4 or4(uint4 x, uint4 y) {
  return make_uint4(x.x | y.x, x.y | y.y, x.z | y.z, x.w | y.w);
}
__device__ __forceinline__ RawKey load_slot(const QueryView& v, const AttnArgs& a, int t, bool live, int j, int g,
                                            int w, int32_t id) {
  // 32-bit throughout: kv_rows < 2^23, win_cap < 2^22.  An entry slot has
  // wi < 0; the unsigned compares take id < 0 and wi < 0 as out of range.
  // The tile's kind is the same in every lane: a tile of entries skips the
  // window offsets and a tile of window tokens the entry offsets (a scalar
  // branch around arithmetic only; the loads below are unconditional).
  const int wi = t * AT_TILE + j - a.k;
  const int tk = tile_kind(t, a.k);
  bool ent = false, win = false;
  uint32_t oc = AT_OOB, os = AT_OOB, ow = AT_OOB;
  if (tk != TK_WINDOW) {
    ent = live && wi < 0 && (uint32_t)id < (uint32_t)a.kv_rows;
    oc = ent ? (uint32_t)id * CODE_BYTES + 64u * w + 16u * g : AT_OOB;
    os = ent ? (uint32_t)id * SCALE_BYTES + 8u * w + 2u * g : AT_OOB;
  }
  if (tk != TK_ENTRY) {
    win = live && (uint32_t)wi < (uint32_t)NWIN && wi >= (NWIN - 1) - v.p;
    // ring row of window token wi: wbase + wi < 2 win_cap, and when it is
    // below win_cap the wrapped difference is the larger
    const uint32_t row0 = (uint32_t)(v.wbase + wi);
    const uint32_t row = __builtin_elementwise_min(row0, row0 - (uint32_t)v.win_cap);
    ow = win ? row * D + AT_QCH * w + 32u * g : AT_OOB;
  }
  const uint4 c = load_b128(v.codes, oc);
  const uint32_t sc = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(v.scales, os, 0, 0);
  const uint4 wa = load_b128(v.win, ow), wb = load_b128(v.win, ow + 16u);
  RawKey r;
  r.a = or4(c, wa);
  r.b = wb;
  r.sc = sc;
  r.kind = ent ? 1 : (win ? 2 : 0);
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
// unnormalized weights stay <= 2^8 and O is rarely rescaled.
constexpr float AT_RESCALE = 8.0f;

// Four fp16 values of one channel across four key rows in LDS: lanes
// 4 r + c of each 16-lane group point at 8 bytes (4 channels) of row r, and
// lane i of the group receives channel i of rows 0 .. 3 (gfx950's
// ds_read_b64_tr_b16).
__device__ __forceinline__ f16x4 lds_read_tr16(const uint8_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// fp16(p0 - hi.x) | fp16(p1 - hi.y) << 16: the lo halves of a hi / lo split
// of two weights whose hi halves are hi, one mixed-precision FMA each
// (v_fma_mix*: source 0 is an fp16 half of hi, the others float32).
__device__ __forceinline__ uint32_t split_lo(f16x2 hi, float p0, float p1) {
  const uint32_t h = __builtin_bit_cast(uint32_t, hi);
  uint32_t lo;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lo) : "v"(h), "v"(p0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(lo) : "v"(h), "v"(p1));
  return lo;
}

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

// Running state of one wave: O of heads 4 g + r (rows) x channels
// 128 w + 16 n + j (acc_o[n][r]); max and sum of head j.
struct AttnState {
  f32x4 acc_o[8];
  float m_run, l_run;
};

__device__ __forceinline__ void state_init(AttnState& st) {
#pragma unroll
  for (int n = 0; n < 8; ++n) st.acc_o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -__builtin_huge_valf();
  st.l_run = 0.f;
}

// Q of head j, channels 128 w + 32 g .. + 31, scaled by the logit factor
// (sm_scale log2 e, so S is in the log2 domain of the softmax) and split into
// fp16 hi / lo halves per k-step.
__device__ __forceinline__ void load_q(const AttnArgs& a, int64_t qi, int j, int g, int w, float4 (&qraw)[8]) {
  const float4* src = reinterpret_cast<const float4*>(a.q + (qi * HEADS + j) * D + AT_QCH * w + 32 * g);
#pragma unroll
  for (int i = 0; i < 8; ++i) qraw[i] = src[i];
}
__device__ __forceinline__ void split_q(const float4 (&qraw)[8], float cq, f16x8 (&qh)[4], f16x8 (&ql)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float4 x = qraw[2 * s], y = qraw[2 * s + 1];
    const float v[8] = {x.x * cq, x.y * cq, x.z * cq, x.w * cq, y.x * cq, y.y * cq, y.z * cq, y.w * cq};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 h = (_Float16)v[e];
      qh[s][e] = h;
      ql[s][e] = (_Float16)(v[e] - (float)h);
    }
  }
}

// Step 2 of one tile for this wave (TK = the tile's kind): the key slices to
// the wave's LDS rows and the wave's partial S^T = K (Q_hi + Q_lo)^T.
template <int TK>
__device__ __forceinline__ f32x4 tile_qk(const RawKey& cur, const f16x8 (&qh)[4], const f16x8 (&ql)[4],
                                         uint8_t* krow, int j, int g) {
  __builtin_amdgcn_wave_barrier();   // the previous tile's LDS reads come first
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f16x8 av = key_slice<TK>(cur, s);
    *reinterpret_cast<f16x8*>(krow + j * AT_KPITCH + 64 * g + 16 * s) = av;
    sc = mfma_f16_16x16x32(av, qh[s], sc);
    sc = mfma_f16_16x16x32(av, ql[s], sc);
  }
  return sc;
}

// Steps 2-4 of one tile for this wave.  krow: the wave's LDS key rows; sbuf:
// the group's partial-S exchange buffer for this tile's parity.  Every wave
// of the block calls this the same number of times (it holds a barrier).
// Only the key conversion depends on the tile kind (a scalar branch).
__device__ __forceinline__ void attn_tile(int tk, AttnState& st, const RawKey& cur, const f16x8 (&qh)[4],
                                          const f16x8 (&ql)[4], uint8_t* krow, f32x4 (*sbuf)[64], int w,
                                          int lane, int j, int g) {
  f32x4 part;
  if (tk == TK_ENTRY) part = tile_qk<TK_ENTRY>(cur, qh, ql, krow, j, g);
  else if (tk == TK_WINDOW) part = tile_qk<TK_WINDOW>(cur, qh, ql, krow, j, g);
  else part = tile_qk<TK_MIXED>(cur, qh, ql, krow, j, g);
  sbuf[w][lane] = part;
  __syncthreads();
  f32x4 S = sbuf[0][lane];
#pragma unroll
  for (int v = 1; v < AT_WAVES; ++v) {
    const f32x4 o = sbuf[v][lane];
    S[0] += o[0]; S[1] += o[1]; S[2] += o[2]; S[3] += o[3];
  }

  // ---- 3. online softmax (lane: keys 4g+r, head j), lazy rescaling --------
  const uint32_t vmask = (uint32_t)(__ballot(cur.kind != 0) & 0xFFFFull);
  float x[4] = {S[0], S[1], S[2], S[3]};
  if (vmask != 0xFFFFu) {   // wave-uniform: only tiles with an absent key mask
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = ((vmask >> (4 * g + r)) & 1u) ? x[r] : -__builtin_huge_valf();
  }
  float mx = fmax_nn(fmax_nn(x[0], x[1]), fmax_nn(x[2], x[3]));
  mx = max_xor32(max_xor16(mx));
  const bool first = (st.m_run == -__builtin_huge_valf());
  const bool move = !first && (mx > st.m_run + AT_RESCALE);
  if (__ballot(move)) {
    const float alpha = move ? exp2_loop(st.m_run - mx) : 1.0f;
    st.l_run *= alpha;
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      st.acc_o[n][0] *= al[0]; st.acc_o[n][1] *= al[1];
      st.acc_o[n][2] *= al[2]; st.acc_o[n][3] *= al[3];
    }
  }
  if (first || move) st.m_run = mx;
  const float base = (st.m_run == -__builtin_huge_valf()) ? 0.f : st.m_run;
  // A operands of P V: P_hi and P_lo of keys 4g..4g+3 (head j).  hi + lo
  // holds each weight to ~2^-22, so the sum takes the float32 weights.
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = exp2_loop(x[r] - base);
  const float psum = (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const f16x2 h01 = {(_Float16)pr[0], (_Float16)pr[1]}, h23 = {(_Float16)pr[2], (_Float16)pr[3]};
  const f16x4 ph = {h01[0], h01[1], h23[0], h23[1]};
  const f16x4 pl = __builtin_bit_cast(f16x4, make_uint2(split_lo(h01, pr[0], pr[1]), split_lo(h23, pr[2], pr[3])));
  st.l_run += psum;   // this lane's keys only; the four lanes of head j are summed at the end

  // ---- 4. P V: B operands straight from the key rows in LDS ----------------
  // A transposed read (ds_read_b64_tr_b16) hands lane (i, g) channel
  // 16 n + i of keys 4g .. 4g+3 when lanes 4 r + c of its 16-lane group point
  // at key 4g + r, channels 16 n + 4c .. + 3 (8 bytes of one row).
  const uint8_t* vrow = krow + (4 * g + (j >> 2)) * AT_KPITCH + 8 * (j & 3);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const f16x4 b = lds_read_tr16(vrow + 32 * n);
    st.acc_o[n] = mfma_f16_16x16x16(ph, b, st.acc_o[n]);
    st.acc_o[n] = mfma_f16_16x16x16(pl, b, st.acc_o[n]);
  }
}

// Merge the KG groups' states (group 0 keeps the result; the others return
// false) and write the block's result: the output when the query has one
// split, else the split's partial (O unnormalized, max, sum).
template <int KG, class Lds>
__device__ __forceinline__ void attn_finish(Lds& lds, AttnState& st, const AttnArgs& a, int64_t qi,
                                            int split, int kg, int w, int lane, int j, int g) {
  st.l_run = sum_xor32(sum_xor16(st.l_run));   // head j's sum over all keys of this group
  // lane holds O[head 4g + r][channel 128 w + 8 j + n]; m_run, l_run are head j's
  float lsum[4];   // sum of head 4 g + r over the groups
  if constexpr (KG > 1) {
    __syncthreads();                                   // loop LDS is free
    if (w == 0 && lane < 16) {
      lds.red.ml[kg][0][j] = st.m_run;
      lds.red.ml[kg][1][j] = st.l_run;
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
      st.m_run = M;
      st.l_run = L;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      st.acc_o[n][0] *= mine[0]; st.acc_o[n][1] *= mine[1];
      st.acc_o[n][2] *= mine[2]; st.acc_o[n][3] *= mine[3];
    }
    if (kg > 0) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) lds.red.o[kg - 1][w][4 * n + r][lane] = st.acc_o[n][r];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int v = 0; v < KG - 1; ++v)
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc_o[n][r] += lds.red.o[v][w][4 * n + r][lane];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = __shfl(st.l_run, 4 * g + r);
  }

  if (a.n_splits == 1) {
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) inv[r] = lsum[r] > 0.f ? 1.0f / lsum[r] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = a.out + (qi * HEADS + 4 * g + r) * D + AT_QCH * w + j;
#pragma unroll
      for (int n = 0; n < 8; ++n) dst[16 * n] = st.acc_o[n][r] * inv[r];
    }
  } else {
    const int64_t ps = qi * a.n_splits + split;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = a.part_o + (ps * HEADS + 4 * g + r) * D + AT_QCH * w + j;
#pragma unroll
      for (int n = 0; n < 8; ++n) dst[16 * n] = st.acc_o[n][r];
    }
    if (w == 0 && lane < 16) {
      a.part_ml[(ps * 2 + 0) * HEADS + j] = st.m_run;
      a.part_ml[(ps * 2 + 1) * HEADS + j] = st.l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// Key loaders of a block whose slots are all selected entries (PATH_ENTRY)
// or all window tokens (PATH_WINDOW): only that kind of bytes is loaded.
constexpr int PATH_ENTRY = 0, PATH_WINDOW = 1;

// The lane's QK bytes of key slot `slot` (channels 128 w + 32 g .. + 31);
// entries are slots 0 .. k-1, window token i is slot k + i.
template <int PATH>
__device__ __forceinline__ RawKey load_slot_p(const QueryView& v, const AttnArgs& a, int slot, bool live, int g,
                                              int w, int32_t id) {
  RawKey r;
  r.a = make_uint4(0u, 0u, 0u, 0u);
  r.b = make_uint4(0u, 0u, 0u, 0u);
  r.sc = 0u;
  if constexpr (PATH == PATH_ENTRY) {
    const bool ent = live && slot < a.k && id >= 0 && id < a.kv_rows;
    const uint32_t oc = ent ? (uint32_t)id * CODE_BYTES + 64u * w + 16u * g : AT_OOB;
    const uint32_t os = ent ? (uint32_t)id * SCALE_BYTES + 8u * w + 2u * g : AT_OOB;
    r.a = load_b128(v.codes, oc);
    r.sc = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(v.scales, os, 0, 0);
    r.kind = ent ? 1 : 0;
  } else {
    const int wi = slot - a.k;
    const bool win = live && wi >= 0 && wi < NWIN && v.p - (NWIN - 1) + wi >= 0;
    int row = v.wbase + wi;
    row = row >= v.win_cap ? row - v.win_cap : row;
    const uint32_t ow = win ? (uint32_t)row * D + AT_QCH * w + 32u * g : AT_OOB;
    r.a = load_b128(v.win, ow);
    r.b = load_b128(v.win, ow + 16u);
    r.kind = win ? 2 : 0;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Pair kernel (decode batches): block (query, split) of four waves -- wave w
// owns channels 128 w .. 128 w + 127 of every key -- takes E pairs of 32
// selected entries (entry pairs split E .. split E + E - 1) and one pair of
// 32 window tokens (window pair `split`; the window's four pairs go to
// splits 0-3), all loaded up front.  Each pair holds one key format, fixed
// at compile time, so no lane carries the registers of both.  The host
// picks E and the number of splits so that the blocks fill the GPU about
// once: a cold gather is bound by the cache lines a compute unit can have
// in flight, so spreading a query over more compute units shortens it.
//
// Key order.  QK runs on two 16-key MFMA tiles per pair; row 4 q + r of tile
// h holds pair key q + 4 (2 r + h) (q, r < 4).  The score fragment of lane
// (j, g) -- rows 4 g .. 4 g + 3 of both tiles, column j -- is then head j
// over the eight pair keys g + 4 m, which is exactly the A operand that lane
// feeds to the 16x16x32 P V product: P never moves between lanes, and P V
// contracts 32 keys per instruction (the 16-key fp16 product runs at half
// the rate on this GPU).
// Per block:
//   1. the pairs' slot ids (one word per lane, each id then read from the
//      lane that loaded it), Q, and per pair the QK bytes (lane (j, g): the
//      key of row j of each tile, its 32 channels -- four lanes read 64
//      contiguous bytes of a row).  Each wave passes its bytes through its
//      own LDS rows into the P V layout (lane (c, g): the keys g + 4 m,
//      channels 128 w + 8 c .. + 7), so a key is read from memory once and
//      a wave has few enough loads to keep them all in flight;
//   2. partial S over the wave's channels for every pair -> LDS; barrier;
//   3. wave p % 4 sums the four partials of pair p (in wave order) and
//      publishes the pair's head maxima; barrier;
//   4. the same wave forms P = 2^(S - M) of pair p against the block's head
//      maxima M, splits it into fp16 hi / lo halves and publishes both with
//      the pair's head sums; barrier;
//   5. every wave: P V over all pairs, the hi products of a pair before its
//      lo products (an accumulator's two updates are eight MFMAs apart).
constexpr int AT_PAIR = 32;
constexpr int AT_WIN_PAIRS = NWIN / AT_PAIR;   // window pairs (one per split 0-3)
static_assert(NWIN % AT_PAIR == 0, "the window is whole pairs");
constexpr int AT_E_MAX = 4;                    // entry pairs per block, at most

template <int NP>
struct PairLds {
  f32x4 s[NP][AT_WAVES][2][64];   // partial S^T fragments (tile 0, tile 1) per wave
  f16x8 p[NP][2][64];             // P of every pair as A operands: hi, lo
  float pmax[NP][HEADS];          // head maxima of each pair
  float psum[NP][HEADS];          // head sums of each pair's weights
};

// Row i < 16 of QK tile h of a pair is pair key (i >> 2) + 4 (2 (i & 3) + h).
__device__ __forceinline__ int pair_row_key(int h, int i) { return (i >> 2) + 4 * (2 * (i & 3) + h); }
// Element kk < 8 of lane group g's P V operands (tile kk >> 2, row
// 4 g + (kk & 3)): pair key g + 4 (2 (kk & 3) + (kk >> 2)).
__device__ __forceinline__ int pair_v_key(int g, int kk) { return pair_row_key(kk >> 2, 4 * g + (kk & 3)); }

// One wave's LDS rows for turning the QK layout into the P V layout: per
// entry pair the wave's 64 code bytes and 8 scale bytes of each key, and
// the wave's 128 bytes of each window token.
template <int E>
struct PairStage {
  uint8_t code[E][AT_PAIR][64];
  uint8_t scale[E][AT_PAIR][8];
  uint8_t win[AT_PAIR][128];
};

// Key slot of key 0 of pair p of a block: entries are slots 0 .. k-1 (entry
// pair e holds slots 32 e ..), window token i is slot k + i.
template <int E>
__device__ __forceinline__ int pair_slot0(const AttnArgs& a, int split, int p) {
  return p < E ? AT_PAIR * (split * E + p) : a.k + AT_PAIR * split;
}

// P V bytes of one key (lane column c, wave w): channels 128 w + 8 c .. + 7 --
// four E2M1 code bytes and the E4M3 scale of their 16-channel group, or
// eight E4M3 window bytes.  An absent key holds zeros (its QK loads read
// past the views).
struct RawV {
  uint32_t c;    // codes, or window bytes 0-3
  uint32_t w1;   // window bytes 4-7
  uint32_t sc;   // scale byte (entries)
};

// stage_*: the QK bytes lane (j, g) loaded for pair key K to the wave's LDS
// rows; unstage_*: the P V bytes of pair key K for lane (c, g) -- four code
// bytes and the scale byte of channels 128 w + 8 c .. + 7, or eight window
// bytes.  LDS operations of one wave complete in order, so no barrier is
// needed between the two.
template <int E>
__device__ __forceinline__ void stage_entry(PairStage<E>& st, int p, int K, int g, const RawKey& r) {
  *reinterpret_cast<uint4*>(&st.code[p][K][16 * g]) = r.a;
  *reinterpret_cast<uint16_t*>(&st.scale[p][K][2 * g]) = (uint16_t)r.sc;
}
template <int E>
__device__ __forceinline__ void stage_window(PairStage<E>& st, int K, int g, const RawKey& r) {
  *reinterpret_cast<uint4*>(&st.win[K][32 * g]) = r.a;
  *reinterpret_cast<uint4*>(&st.win[K][32 * g + 16]) = r.b;
}
template <int E>
__device__ __forceinline__ RawV unstage_entry(const PairStage<E>& st, int p, int K, int c) {
  RawV r;
  r.c = *reinterpret_cast<const uint32_t*>(&st.code[p][K][4 * c]);
  r.w1 = 0u;
  r.sc = st.scale[p][K][c >> 1];
  return r;
}
template <int E>
__device__ __forceinline__ RawV unstage_window(const PairStage<E>& st, int K, int c) {
  const uint2 x = *reinterpret_cast<const uint2*>(&st.win[K][8 * c]);
  RawV r;
  r.c = x.x;
  r.w1 = x.y;
  r.sc = 0u;
  return r;
}

// The eight B operands of a pair's P V (N-tile n: channel 128 w + 8 c + n of
// the lane's pair keys) from its eight RawV (element kk: pair_v_key(g, kk)).
// Entry bytes widen with scale 1 and are multiplied by the group scale in
// fp16 (E2M1 x E4M3 has at most 5 significant bits: exact).
template <int PATH>
__device__ __forceinline__ void pair_v_operands(const RawV (&rv)[8], f16x8 (&vb)[8]) {
  uint32_t wv[8][4];   // key kk: channels (2 b, 2 b + 1) as an fp16 pair, b < 4
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    f16x2 e[4];
    if constexpr (PATH == PATH_ENTRY) {
      const _Float16 s = fp8x2_to_f16<0>(rv[kk].sc)[0];
      const f16x2 sp = f16x2{s, s};
      e[0] = fp4x2_to_f16<0>(rv[kk].c) * sp;
      e[1] = fp4x2_to_f16<1>(rv[kk].c) * sp;
      e[2] = fp4x2_to_f16<2>(rv[kk].c) * sp;
      e[3] = fp4x2_to_f16<3>(rv[kk].c) * sp;
    } else {
      e[0] = fp8x2_to_f16<0>(rv[kk].c);
      e[1] = fp8x2_to_f16<1>(rv[kk].c);
      e[2] = fp8x2_to_f16<0>(rv[kk].w1);
      e[3] = fp8x2_to_f16<1>(rv[kk].w1);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) wv[kk][b] = f16x2_bits(e[b]);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t lo[4], hi[4];   // channel 2 b / 2 b + 1 of key pairs (2 i, 2 i + 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = __builtin_amdgcn_perm(wv[2 * i + 1][b], wv[2 * i][b], 0x05040100u);
      hi[i] = __builtin_amdgcn_perm(wv[2 * i + 1][b], wv[2 * i][b], 0x07060302u);
    }
    vb[2 * b] = __builtin_bit_cast(f16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
    vb[2 * b + 1] = __builtin_bit_cast(f16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
  }
}

template <int E>
__global__ __launch_bounds__(AT_THREADS) void attn_pair_kernel(AttnArgs a) {
  constexpr int NP = E + 1;   // E entry pairs, then the window pair
  __shared__ __attribute__((aligned(16))) PairLds<NP> lds;
  __shared__ __attribute__((aligned(16))) PairStage<E> stage_all[AT_WAVES];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int64_t qi = blockIdx.x;   // query in x: see attn_grid
  const int split = blockIdx.y;
  if (qi >= a.n_queries) return;  // grid padding (the whole block)
  const QueryView v = query_view(a, qi);

  // ---- 1. loads ---------------------------------------------------------------
  // slot ids: lane l holds key l % 32 of entry pair 2 i + l / 32
  constexpr int NI = (E + 1) / 2;
  int32_t ids[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = 2 * i + (lane >> 5);
    ids[i] = slot_id(v, a.k, 0, p < E, AT_PAIR * (split * E + p) + (lane & 31));
  }
  // the window pair's QK bytes and Q do not wait for the ids
  RawKey rk[NP][2];
  const int wbase = pair_slot0<E>(a, split, E);
#pragma unroll
  for (int h = 0; h < 2; ++h) rk[E][h] = load_slot_p<PATH_WINDOW>(v, a, wbase + pair_row_key(h, j), true, g, w, -1);
  float4 qraw[8];
  load_q(a, qi, j, g, w, qraw);
  uint32_t vbits[NP];   // bit kk: pair key pair_v_key(g, kk) is present
#pragma unroll
  for (int p = 0; p < E; ++p) {
    const int base = pair_slot0<E>(a, split, p);
    const int32_t id = ids[p >> 1];
    const bool ok = base + (lane & 31) < a.k && id >= 0 && id < a.kv_rows;
    const uint32_t vm = (uint32_t)(__ballot(ok) >> (32 * (p & 1)));   // bit K: pair key K
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int K = pair_row_key(h, j);
      const int32_t idk = __shfl(id, K + 32 * (p & 1));
      rk[p][h] = load_slot_p<PATH_ENTRY>(v, a, base + K, true, g, w, idk);
    }
    vbits[p] = 0u;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) vbits[p] |= ((vm >> pair_v_key(g, kk)) & 1u) << kk;
  }
  {
    vbits[E] = 0u;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int wi = wbase + pair_v_key(g, kk) - a.k;
      const bool ok = wi >= 0 && wi < NWIN && v.p - (NWIN - 1) + wi >= 0;
      vbits[E] |= (ok ? 1u : 0u) << kk;
    }
  }
  // P V bytes through the wave's LDS rows
  PairStage<E>& stg = stage_all[w];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int K = pair_row_key(h, j);
#pragma unroll
    for (int p = 0; p < E; ++p) stage_entry<E>(stg, p, K, g, rk[p][h]);
    stage_window<E>(stg, K, g, rk[E][h]);
  }
  RawV rv[NP][8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int K = pair_v_key(g, kk);
#pragma unroll
    for (int p = 0; p < E; ++p) rv[p][kk] = unstage_entry<E>(stg, p, K, j);
    rv[E][kk] = unstage_window<E>(stg, K, j);
  }
  f16x8 qh[4], ql[4];
  split_q(qraw, a.c_log2, qh, ql);

  // ---- 2. partial S^T of every pair ------------------------------------------------
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 av = p < E ? entry_slice(rk[p][h], s) : window_slice(rk[p][h], s);
        sc = mfma_f16_16x16x32(av, qh[s], sc);
        sc = mfma_f16_16x16x32(av, ql[s], sc);
      }
      lds.s[p][w][h][lane] = sc;
    }
  }
  __syncthreads();

  // ---- 3. wave p % 4: the scores of pair p and their head maxima -------------------
  constexpr int MINE = (NP + AT_WAVES - 1) / AT_WAVES;   // pairs per wave, at most
  float x[MINE][8];
#pragma unroll
  for (int m = 0; m < MINE; ++m) {
    const int p = w + AT_WAVES * m;   // wave-uniform
    if (p < NP) {
      uint32_t vb_p = vbits[0];
#pragma unroll
      for (int q = 1; q < NP; ++q) vb_p = q == p ? vbits[q] : vb_p;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 S = lds.s[p][0][h][lane];
#pragma unroll
        for (int vv = 1; vv < AT_WAVES; ++vv) {
          const f32x4 o = lds.s[p][vv][h][lane];
          S[0] += o[0]; S[1] += o[1]; S[2] += o[2]; S[3] += o[3];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) x[m][4 * h + r] = S[r];
      }
      // x[m][kk] (tile kk >> 2, row 4 g + (kk & 3)) is pair key
      // pair_v_key(g, kk), whose presence is bit kk of the pair's vbits
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) x[m][kk] = ((vb_p >> kk) & 1u) ? x[m][kk] : -__builtin_huge_valf();
      float mx = fmax_nn(fmax_nn(fmax_nn(x[m][0], x[m][1]), fmax_nn(x[m][2], x[m][3])),
                         fmax_nn(fmax_nn(x[m][4], x[m][5]), fmax_nn(x[m][6], x[m][7])));
      mx = max_xor32(max_xor16(mx));
      if (g == 0) lds.pmax[p][j] = mx;
    }
  }
  __syncthreads();

  // ---- 4. P of the wave's pairs against the block's head maxima --------------------
  float M = lds.pmax[0][j];
#pragma unroll
  for (int p = 1; p < NP; ++p) M = fmax_nn(M, lds.pmax[p][j]);
  const float base = (M == -__builtin_huge_valf()) ? 0.f : M;
#pragma unroll
  for (int m = 0; m < MINE; ++m) {
    const int p = w + AT_WAVES * m;
    if (p < NP) {
      float pr[8];   // <= 1; 0 for an absent key
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) pr[kk] = exp2_loop(x[m][kk] - base);
      f16x2 hv[4];
      uint32_t lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[i] = f16x2{(_Float16)pr[2 * i], (_Float16)pr[2 * i + 1]};
        lv[i] = split_lo(hv[i], pr[2 * i], pr[2 * i + 1]);
      }
      const f16x8 ph = {hv[0][0], hv[0][1], hv[1][0], hv[1][1], hv[2][0], hv[2][1], hv[3][0], hv[3][1]};
      const f16x8 pl = __builtin_bit_cast(f16x8, make_uint4(lv[0], lv[1], lv[2], lv[3]));
      // the float32 weights, which P_hi + P_lo match to ~2^-22
      float psum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      psum = sum_xor32(sum_xor16(psum));
      lds.p[p][0][lane] = ph;
      lds.p[p][1][lane] = pl;
      if (g == 0) lds.psum[p][j] = psum;
    }
  }
  __syncthreads();

  // ---- 5. P V over all pairs ----------------------------------------------------------
  f32x4 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    f16x8 vb[8];
    if (p < E) pair_v_operands<PATH_ENTRY>(rv[p], vb);
    else pair_v_operands<PATH_WINDOW>(rv[p], vb);
    const f16x8 ph = lds.p[p][0][lane], pl = lds.p[p][1][lane];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = mfma_f16_16x16x32(ph, vb[n], acc[n]);
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = mfma_f16_16x16x32(pl, vb[n], acc[n]);
  }

  // ---- result: O of heads 4 g + r, channels 128 w + 8 j + n --------------------------
  float lsum[4], mrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    float L = lds.psum[0][h], Mh = lds.pmax[0][h];
#pragma unroll
    for (int p = 1; p < NP; ++p) {
      L += lds.psum[p][h];
      Mh = fmax_nn(Mh, lds.pmax[p][h]);
    }
    lsum[r] = L;
    mrow[r] = Mh;
  }
  if (a.n_splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv = lsum[r] > 0.f ? 1.0f / lsum[r] : 0.f;
      float4* dst = reinterpret_cast<float4*>(a.out + (qi * HEADS + 4 * g + r) * D + AT_QCH * w + 8 * j);
      dst[0] = make_float4(acc[0][r] * inv, acc[1][r] * inv, acc[2][r] * inv, acc[3][r] * inv);
      dst[1] = make_float4(acc[4][r] * inv, acc[5][r] * inv, acc[6][r] * inv, acc[7][r] * inv);
    }
  } else {
    // partials: buffer stores with the non-temporal policy (the combine reads
    // them once; measured 0.5 us faster per 128K layer than plain stores)
    constexpr int NT_POLICY = 2;
    const int64_t ps = qi * a.n_splits + split;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.part_o + ps * HEADS * D), (short)0, HEADS * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.part_ml + ps * 2 * HEADS), (short)0, 2 * HEADS * 4, 0x00020000);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = (uint32_t)(((4 * g + r) * D + AT_QCH * w + 8 * j) * 4);
      const i32x4 lo = {(int)__float_as_uint(acc[0][r]), (int)__float_as_uint(acc[1][r]),
                        (int)__float_as_uint(acc[2][r]), (int)__float_as_uint(acc[3][r])};
      const i32x4 hi = {(int)__float_as_uint(acc[4][r]), (int)__float_as_uint(acc[5][r]),
                        (int)__float_as_uint(acc[6][r]), (int)__float_as_uint(acc[7][r])};
      __builtin_amdgcn_raw_buffer_store_b128(lo, ro, off, 0, NT_POLICY);
      __builtin_amdgcn_raw_buffer_store_b128(hi, ro, off + 16u, 0, NT_POLICY);
    }
    if (w == 0 && j == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        __builtin_amdgcn_raw_buffer_store_b32((int)__float_as_uint(mrow[r]), rm, (uint32_t)((4 * g + r) * 4), 0,
                                              NT_POLICY);
        __builtin_amdgcn_raw_buffer_store_b32((int)__float_as_uint(lsum[r]), rm,
                                              (uint32_t)((HEADS + 4 * g + r) * 4), 0, NT_POLICY);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stream kernel: block (split, query) of KG key groups walks the split's
// tiles t_begin + kg + KG i; key bytes DEPTH tiles ahead, slot ids 2 DEPTH
// ahead.  One group: four waves per SIMD (registers capped at 128, no
// spills); two groups (two tiles in flight): three waves per SIMD.
template <int KG> constexpr int stream_depth() { return KG == 1 ? 1 : 2; }

template <int KG>
__global__ __launch_bounds__(AT_THREADS * KG) __attribute__((amdgpu_waves_per_eu(KG == 1 ? 4 : 3))) void attn_stream_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnLds<KG> lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = (tid >> 6) & (AT_WAVES - 1);
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 8);
  constexpr int DEPTH = stream_depth<KG>();
  const int j = lane & 15, g = lane >> 4;
  const int64_t qi = blockIdx.x;   // query in x: see attn_grid
  const int split = blockIdx.y;
  if (qi >= a.n_queries) return;  // grid padding (the whole block)
  const int n_tiles = (a.k + NWIN + AT_TILE - 1) / AT_TILE;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  t_end = t_end < n_tiles ? t_end : n_tiles;
  // group kg takes tiles t_begin + kg + KG i; every group runs n_iter rounds
  // (a round past t_end is all padding), so the block barriers line up
  const int n_iter = (t_end - t_begin + KG - 1) / KG;
  auto tile = [&](int i) { return t_begin + kg + KG * i; };

  const QueryView v = query_view(a, qi);
  int32_t id0[DEPTH], id_ahead[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) id0[i] = slot_id(v, a.k, tile(i), tile(i) < t_end, j);
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) id_ahead[i] = slot_id(v, a.k, tile(DEPTH + i), tile(DEPTH + i) < t_end, j);
  float4 qraw[8];
  load_q(a, qi, j, g, w, qraw);
  RawKey ring[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) ring[i] = load_slot(v, a, tile(i), tile(i) < t_end, j, g, w, id0[i]);
  f16x8 qh[4], ql[4];
  split_q(qraw, a.c_log2, qh, ql);

  AttnState st;
  state_init(st);
  uint8_t* krow = lds.loop.k[AT_WAVES * kg + w];
  for (int it = 0; it < n_iter; ++it) {
    const RawKey cur = ring[0];
#pragma unroll
    for (int i = 0; i + 1 < DEPTH; ++i) ring[i] = ring[i + 1];
    const int tn = tile(it + DEPTH);
    ring[DEPTH - 1] = load_slot(v, a, tn, tn < t_end, j, g, w, id_ahead[0]);
#pragma unroll
    for (int i = 0; i + 1 < DEPTH; ++i) id_ahead[i] = id_ahead[i + 1];
    const int ti = tile(it + 2 * DEPTH);
    id_ahead[DEPTH - 1] = slot_id(v, a.k, ti, ti < t_end, j);
    attn_tile(tile_kind(tile(it), a.k), st, cur, qh, ql, krow, lds.loop.s[it & 1][kg], w, lane, j, g);
  }
  attn_finish<KG>(lds, st, a, qi, split, kg, w, lane, j, g);
}

// out[q, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.  One block of
// 128 threads per (query, head), 4 channels per thread; all split loads are
// issued before any use (the splits are independent).
constexpr int AT_MAX_SPLITS = 16;

__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, int64_t n_queries,
                                                           float* __restrict__ out) {
  const int64_t qi = blockIdx.x;   // query in x: see attn_grid
  const int h = blockIdx.y;
  if (qi >= n_queries) return;
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

// XCD-aware grid: the hardware hands workgroups to the eight XCDs round
// robin by linear workgroup id (x fastest), and each XCD has its own L2.
// With the query in x and x padded to a multiple of 8, linear id
// y * gridDim.x + x falls on XCD x % 8 for every y: all splits of a query
// (and, in the combine, all its heads) run on one XCD, so the query's Q is
// fetched from HBM once and re-read from that L2, the split partials are
// read back by the combine from the same L2, and the selection kernels
// (one block per query, x = query) left the query's ids in it too.
dim3 attn_grid(int64_t Q, int y) {
  const int64_t xq = (Q + 7) / 8 * 8;
  return dim3((unsigned)xq, (unsigned)y);
}

// Launch plan.  kind 0: pair kernel (e entry pairs + one window pair per
// block, all loaded up front); kind 1: stream kernel.
struct AttnPlan {
  int kind, kg, e, n_splits, tiles_per_split;
};

// Below 512 queries (decode batches) the pair kernel takes a query in
// max(4, ceil(k / 32e)) splits of e entry pairs (the window's four pairs go
// to splits 0-3), with e chosen so that the Q x splits blocks fill the GPU
// about once (e <= AT_E_MAX, splits <= AT_MAX_SPLITS: k up to 2,048).
// Longer selections stream in 4 splits of two groups.  From 512 queries on
// (prefill) one group streams every tile of its query (no partials).
AttnPlan attn_plan(int64_t Q, int32_t k) {
  const int n_tiles = (k + NWIN + AT_TILE - 1) / AT_TILE;
  AttnPlan pl;
  if (Q < 512) {
    const int n_e = (k + AT_PAIR - 1) / AT_PAIR;
    int want = (int)((256 + Q - 1) / Q);
    want = want < AT_WIN_PAIRS ? AT_WIN_PAIRS : (want > AT_MAX_SPLITS ? AT_MAX_SPLITS : want);
    int e = (n_e + want - 1) / want;
    e = e < 1 ? 1 : (e > AT_E_MAX ? AT_E_MAX : e);
    int s = (n_e + e - 1) / e;
    s = s < AT_WIN_PAIRS ? AT_WIN_PAIRS : s;
    if (s <= AT_MAX_SPLITS) {
      pl.kind = 0;
      pl.kg = 1;
      pl.e = e;
      pl.tiles_per_split = 0;
      pl.n_splits = s;
      return pl;
    }
  }
  int kg = 1, want = 1;
  if (Q < 512) {
    kg = 2;
    want = 4;
  }
  int max_split = n_tiles / kg;
  max_split = max_split < 1 ? 1 : max_split;
  max_split = max_split < AT_MAX_SPLITS ? max_split : AT_MAX_SPLITS;
  int s = want < max_split ? want : max_split;
  s = s < 1 ? 1 : s;
  pl.kind = 1;
  pl.kg = kg;
  pl.e = 0;
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
  a.n_queries = Q;
  const dim3 grid = attn_grid(Q, a.n_splits);
  if (pl.kind == 0) {
    switch (pl.e) {
      case 1: hipLaunchKernelGGL(attn_pair_kernel<1>, grid, dim3(AT_THREADS), 0, st, a); break;
      case 2: hipLaunchKernelGGL(attn_pair_kernel<2>, grid, dim3(AT_THREADS), 0, st, a); break;
      case 3: hipLaunchKernelGGL(attn_pair_kernel<3>, grid, dim3(AT_THREADS), 0, st, a); break;
      default: hipLaunchKernelGGL(attn_pair_kernel<AT_E_MAX>, grid, dim3(AT_THREADS), 0, st, a); break;
    }
  }
  else if (pl.kg == 2)
    hipLaunchKernelGGL(attn_stream_kernel<2>, grid, dim3(AT_THREADS * 2), 0, st, a);
  else
    hipLaunchKernelGGL(attn_stream_kernel<1>, grid, dim3(AT_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, attn_grid(Q, HEADS), dim3(128), 0, st, a.part_o, a.part_ml, a.n_splits,
                     Q, out);
  return hipGetLastError();
}

}  // namespace csa

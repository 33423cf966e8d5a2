// C-ABI entry points of libcsa: host-side validation, workspace layout and
// launch sequencing.  No entry point here allocates, frees or synchronizes;
// every check runs before the first launch, so an error enqueues nothing.
// (The global-KV file pair in kvio.hip blocks on its copies and file I/O.)
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"
#include "kernels.h"
#include "status.h"

namespace csa {

namespace {
thread_local std::string g_last_error;
}  // namespace

csa_status fail(csa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

csa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace csa

using namespace csa;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

#define CHECK_PTR(p)                                                                   \
  do {                                                                                 \
    if ((p) == nullptr) return fail(CSA_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);    \
  } while (0)
#define CHECK_ALIGN(p, a)                                                              \
  do {                                                                                 \
    if (!aligned((p), (a)))                                                            \
      return fail(CSA_ERR_ALIGNMENT, "%s: %s is not %d-byte aligned", fn, #p, (int)(a)); \
  } while (0)
#define CHECK(cond, status, ...)                                                       \
  do {                                                                                 \
    if (!(cond)) return fail((status), __VA_ARGS__);                                   \
  } while (0)

// Workspace plan of a layer call: offsets of its scratch buffers.
// Full layers select their Top-K among the entries of the best blocks: the
// top-P blocks by (block max desc, block id asc) contain every Top-K entry
// whenever P >= K (a block ranked above the block of a Top-K entry e has a
// max >= s(e), equality only at a lower block id, whose entry then ties with
// and precedes e).  P is the pool when one is built, else K blocks.
//
// When the pool, top_k and the row fit one block (full_select_supported) the
// Full layer writes no scores at all: the dense scan emits only the block
// maxima, and the fused selection rescores the entries of the top_k blocks.
struct LayerPlan {
  int64_t Q = 0, ncols = 0, nblk = 0;
  size_t off_scores = 0, off_bm = 0, off_blocks = 0, off_sel = 0, off_attn = 0, total = 0;
  bool pooled = false, fused_full = false;
  bool fused_scores = false;   // fused Full layer that gathers the scan's scores
  bool split_full = false;     // fused Full layer whose rescoring runs in a second kernel
  size_t off_split = 0;
};

LayerPlan plan_layer(int32_t mode, const csa_layer_args* a) {
  LayerPlan p;
  p.Q = a->n_seq * a->q_per_seq;
  size_t off = 0;
  if (mode == CSA_MODE_FULL || mode == CSA_MODE_REINDEX) {
    p.pooled = (mode == CSA_MODE_REINDEX) && a->pool_blocks != nullptr;
    p.ncols = p.pooled ? (int64_t)CSA_BLOCK * a->n_pool_blocks : a->n_entries;
    const int32_t nb = a->build_pool ? a->n_pool_blocks : a->top_k;
    p.nblk = (p.ncols + 7) / 8;
    p.fused_full = mode == CSA_MODE_FULL && full_select_supported(p.nblk, nb, a->top_k);
    // The scan can also write every score, so that the fused selection
    // gathers the chosen blocks' scores instead of rescoring their 512 KiB
    // of keys per query.  Small decode batches: one block per query
    // rescoring is ~17 us of latency, but writing the scores beside the
    // HBM-bound decode scan costs it more than their bytes (32 x 1M entries,
    // 32 MiB of scores in whole 256-byte stores: step 0.365 against 0.349 ms
    // with the rescoring; 64 x 128K: -9 us per step), so only batches with at
    // most 2^22 scores take this path.
    // Prefill chunks: the MFMA-bound tile scan absorbs the stores, and the
    // rescoring re-reads 512 KiB of keys per query (2,048 queries at 32K:
    // step 0.352 -> 0.303 ms; 4,096 at 256K, 1.1 GB of scores: 2.918 ->
    // 2.895 ms), so chunks with at most 2^29 scores (2 GiB of workspace)
    // take it too.
    p.fused_scores = p.fused_full && ((p.Q < 512 && p.Q * p.ncols <= ((int64_t)1 << 22)) ||
                                      (p.Q >= 512 && p.Q * p.ncols <= ((int64_t)1 << 29)));
    // The other decode batches rescore the chosen blocks in a second kernel
    // with several blocks per query (one block per query spends ~17 us
    // gathering a query's 512 KiB of keys).
    p.split_full = p.fused_full && !p.fused_scores && p.Q < 512;
    if (!p.fused_full || p.fused_scores) {
      p.off_scores = off;
      off += round_up((size_t)(p.Q * p.ncols) * sizeof(float));
    }
    size_t sel = 0;
    if (mode == CSA_MODE_FULL) {
      p.off_bm = off;
      off += round_up((size_t)(p.Q * p.nblk) * sizeof(float));
      if (!p.fused_full) {
        if (!a->build_pool) {
          p.off_blocks = off;
          off += round_up((size_t)(p.Q * nb) * sizeof(int32_t));
        }
        sel = pool_topk_workspace_bytes(p.Q, p.nblk, nb, a->top_k);
      }
    } else {
      sel = topk_workspace_bytes(p.Q, p.ncols, a->top_k);
    }
    p.off_sel = off;
    off += round_up(sel);
    if (p.split_full) {
      p.off_split = off;
      off += round_up(full_split_workspace_bytes(p.Q, a->top_k));
    }
  }
  p.off_attn = off;
  off += round_up(attn_workspace_bytes(p.Q, a->top_k));
  p.total = off;
  return p;
}

}  // namespace

extern "C" {

const char* csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported size";
    case CSA_ERR_ALIGNMENT: return "misaligned pointer";
    case CSA_ERR_WORKSPACE: return "workspace too small";
    case CSA_ERR_HIP: return "HIP error";
    case CSA_ERR_IO: return "file error";
    default: return "unknown status";
  }
}

const char* csa_last_error(void) { return csa::last_error(); }

int32_t csa_version(void) { return 100; }

// ------------------------------------------------------------------ a2 ----
csa_status csa_quantize(const float* e, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const char* fn = "csa_quantize";
  CHECK(n >= 0, CSA_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (n == 0) return CSA_OK;
  CHECK_PTR(e); CHECK_PTR(codes); CHECK_PTR(scales);
  CHECK_ALIGN(e, 16); CHECK_ALIGN(codes, 16); CHECK_ALIGN(scales, 16);
  return hip_status(launch_quantize(e, n, codes, scales, stream), fn);
}

csa_status csa_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out,
                          hipStream_t stream) {
  const char* fn = "csa_dequantize";
  CHECK(n >= 0, CSA_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (n == 0) return CSA_OK;
  CHECK_PTR(codes); CHECK_PTR(scales); CHECK_PTR(out);
  CHECK_ALIGN(codes, 16); CHECK_ALIGN(scales, 16); CHECK_ALIGN(out, 16);
  return hip_status(launch_dequantize(codes, scales, n, out, stream), fn);
}

// ------------------------------------------------------------- a1 + a2 ----
size_t csa_compress_quant_workspace_size(int64_t n_entries) {
  return n_entries <= 0 ? 0 : compress_workspace_bytes(n_entries);
}

static csa_status check_compress(const char* fn, const float* x, int64_t n_seq, int64_t n_per_seq,
                                 int64_t x_seq_stride, const float* w, const float* rope_cs, int32_t rope_dim,
                                 float eps, uint8_t* codes, uint8_t* scales, int64_t out_seq_stride,
                                 float* e_out, void* ws, size_t ws_bytes) {
  const int64_t n = n_seq * n_per_seq;
  CHECK_PTR(x); CHECK_PTR(w); CHECK_PTR(codes); CHECK_PTR(scales);
  CHECK(rope_dim >= 0 && rope_dim <= D && rope_dim % 2 == 0, CSA_ERR_UNSUPPORTED,
        "%s: rope_dim must be even and in [0, 512] (got %d)", fn, rope_dim);
  CHECK(rope_dim == 0 || rope_cs != nullptr, CSA_ERR_INVALID_ARG, "%s: rope_cs is NULL", fn);
  CHECK(std::isfinite(eps) && eps >= 0.f, CSA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  CHECK(n_seq == 1 || x_seq_stride >= n_per_seq * 4 * D, CSA_ERR_INVALID_ARG,
        "%s: x_seq_stride overlaps the previous sequence", fn);
  CHECK(x_seq_stride % 4 == 0, CSA_ERR_ALIGNMENT, "%s: x_seq_stride must be a multiple of 4", fn);
  CHECK(n_seq == 1 || out_seq_stride >= n_per_seq, CSA_ERR_INVALID_ARG,
        "%s: out_seq_stride must be >= n_per_seq", fn);
  CHECK_ALIGN(x, 16); CHECK_ALIGN(w, 16); CHECK_ALIGN(codes, 16); CHECK_ALIGN(scales, 16);
  if (rope_cs) CHECK_ALIGN(rope_cs, 4);
  if (e_out) CHECK_ALIGN(e_out, 16);
  size_t need = compress_workspace_bytes(n);
  CHECK(ws != nullptr && ws_bytes >= need, CSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  CHECK_ALIGN(ws, 16);
  return CSA_OK;
}

static csa_status check_window_append(const char* fn, const float* x, int64_t n_seq, int64_t n_tok,
                                      int64_t x_seq_stride, const int32_t* pos0, uint8_t* win,
                                      int64_t win_cap) {
  CHECK_PTR(x); CHECK_PTR(pos0); CHECK_PTR(win);
  CHECK(win_cap >= NWIN, CSA_ERR_UNSUPPORTED, "%s: win_cap must be >= 128", fn);
  CHECK(n_tok <= win_cap, CSA_ERR_INVALID_ARG, "%s: n_tok exceeds win_cap", fn);
  CHECK(x_seq_stride % 4 == 0, CSA_ERR_ALIGNMENT, "%s: x_seq_stride must be a multiple of 4", fn);
  CHECK(n_seq == 1 || x_seq_stride >= n_tok * D, CSA_ERR_INVALID_ARG, "%s: x_seq_stride too small", fn);
  CHECK_ALIGN(x, 16); CHECK_ALIGN(pos0, 4); CHECK_ALIGN(win, 16);
  return CSA_OK;
}

csa_status csa_compress_quant(const float* x, int64_t n_seq, int64_t n_per_seq, int64_t x_seq_stride,
                              const float* w, const float* rope_cs, int32_t rope_dim, float eps,
                              uint8_t* codes, uint8_t* scales, int64_t out_seq_stride, float* e_out,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "csa_compress_quant";
  CHECK(n_seq >= 0 && n_per_seq >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n_seq * n_per_seq == 0) return CSA_OK;
  const csa_status st = check_compress(fn, x, n_seq, n_per_seq, x_seq_stride, w, rope_cs, rope_dim, eps, codes,
                                       scales, out_seq_stride, e_out, ws, ws_bytes);
  if (st != CSA_OK) return st;
  return hip_status(launch_compress_quant(x, n_seq, n_per_seq, x_seq_stride, w, rope_cs, rope_dim, eps,
                                          codes, scales, out_seq_stride, e_out, ws, stream), fn);
}

// ------------------------------------------------------------------ a9 ----
csa_status csa_window_append(const float* x, int64_t n_seq, int64_t n_tok, int64_t x_seq_stride,
                             const int32_t* pos0, uint8_t* win, int64_t win_cap, hipStream_t stream) {
  const char* fn = "csa_window_append";
  CHECK(n_seq >= 0 && n_tok >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n_seq * n_tok == 0) return CSA_OK;
  const csa_status st = check_window_append(fn, x, n_seq, n_tok, x_seq_stride, pos0, win, win_cap);
  if (st != CSA_OK) return st;
  return hip_status(launch_window_append(x, n_seq, n_tok, x_seq_stride, pos0, win, win_cap, stream), fn);
}

// ------------------------------- compression and window append, one launch ----
csa_status csa_compress_quant_append(const float* x, int64_t n_seq, int64_t n_per_seq, int64_t x_seq_stride,
                                     const float* w, const float* rope_cs, int32_t rope_dim, float eps,
                                     uint8_t* codes, uint8_t* scales, int64_t out_seq_stride, float* e_out,
                                     void* ws, size_t ws_bytes, const float* xw, int64_t nw_seq, int64_t nw_tok,
                                     int64_t xw_seq_stride, const int32_t* pos0, uint8_t* win, int64_t win_cap,
                                     hipStream_t stream) {
  const char* fn = "csa_compress_quant_append";
  CHECK(n_seq >= 0 && n_per_seq >= 0 && nw_seq >= 0 && nw_tok >= 0, CSA_ERR_INVALID_ARG, "%s: negative size",
        fn);
  const bool comp = n_seq * n_per_seq > 0, app = nw_seq * nw_tok > 0;
  if (comp) {
    const csa_status st = check_compress(fn, x, n_seq, n_per_seq, x_seq_stride, w, rope_cs, rope_dim, eps, codes,
                                         scales, out_seq_stride, e_out, ws, ws_bytes);
    if (st != CSA_OK) return st;
  }
  if (app) {
    const csa_status st = check_window_append(fn, xw, nw_seq, nw_tok, xw_seq_stride, pos0, win, win_cap);
    if (st != CSA_OK) return st;
  }
  if (!comp && !app) return CSA_OK;
  const WindowAppendArgs ap{xw, nw_seq, nw_tok, xw_seq_stride, pos0, win, win_cap};
  if (!comp) return hip_status(launch_window_append(xw, nw_seq, nw_tok, xw_seq_stride, pos0, win, win_cap, stream), fn);
  return hip_status(launch_compress_quant(x, n_seq, n_per_seq, x_seq_stride, w, rope_cs, rope_dim, eps, codes,
                                          scales, out_seq_stride, e_out, ws, stream, app ? &ap : nullptr),
                    fn);
}

csa_status csa_window_rebuild(const float* x, int64_t n_ring, int64_t n_tok, int64_t x_ring_stride,
                              const int32_t* p_last, uint8_t* win, int64_t win_cap, hipStream_t stream) {
  const char* fn = "csa_window_rebuild";
  CHECK(n_ring >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n_ring == 0) return CSA_OK;
  CHECK_PTR(x); CHECK_PTR(p_last); CHECK_PTR(win);
  CHECK(win_cap >= NWIN && win_cap < ((int64_t)1 << 24), CSA_ERR_UNSUPPORTED, "%s: win_cap must be in [128, 2^24)",
        fn);
  CHECK(n_tok >= 1 && n_tok <= win_cap, CSA_ERR_INVALID_ARG, "%s: need 1 <= n_tok <= win_cap", fn);
  CHECK(x_ring_stride % 4 == 0, CSA_ERR_ALIGNMENT, "%s: x_ring_stride must be a multiple of 4", fn);
  CHECK(n_ring == 1 || x_ring_stride >= n_tok * D, CSA_ERR_INVALID_ARG, "%s: x_ring_stride too small", fn);
  CHECK(n_ring * win_cap < ((int64_t)1 << 26), CSA_ERR_UNSUPPORTED, "%s: too many ring rows", fn);
  CHECK_ALIGN(x, 16); CHECK_ALIGN(p_last, 4); CHECK_ALIGN(win, 16);
  return hip_status(launch_window_rebuild(x, n_ring, n_tok, x_ring_stride, p_last, win, win_cap, stream), fn);
}

// ------------------------------------------------------------------ a3 ----
static csa_status check_score(const char* fn, const ScoreArgs& s) {
  CHECK(s.n_seq >= 0 && s.q_per_seq >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK_PTR(s.q_fp8); CHECK_PTR(s.w); CHECK_PTR(s.q_pos); CHECK_PTR(s.k_fp8);
  CHECK(s.n_entries >= 0 && s.n_entries <= s.k_rows, CSA_ERR_INVALID_ARG,
        "%s: need 0 <= n_entries <= k_rows (%lld, %lld)", fn, (long long)s.n_entries, (long long)s.k_rows);
  CHECK(s.n_entries < (int64_t)1 << 30, CSA_ERR_UNSUPPORTED, "%s: n_entries too large", fn);
  if (s.pool) {
    CHECK(s.n_pool_blocks >= 1 && s.n_pool_blocks <= 65536, CSA_ERR_UNSUPPORTED,
          "%s: n_pool_blocks out of range", fn);
    CHECK(s.block_max == nullptr, CSA_ERR_INVALID_ARG, "%s: block_max is for dense mode only", fn);
    CHECK_ALIGN(s.pool, 4);
  }
  CHECK(s.scores != nullptr || s.block_max != nullptr, CSA_ERR_INVALID_ARG,
        "%s: scores and block_max are both NULL", fn);
  CHECK_ALIGN(s.q_fp8, 16); CHECK_ALIGN(s.k_fp8, 16); CHECK_ALIGN(s.w, 4); CHECK_ALIGN(s.q_pos, 4);
  if (s.scores) CHECK_ALIGN(s.scores, 4);
  if (s.block_max) CHECK_ALIGN(s.block_max, 4);
  return CSA_OK;
}

csa_status csa_index_score(const uint8_t* q_fp8, const float* w, const int32_t* q_pos, int64_t n_seq,
                           int64_t q_per_seq, const uint8_t* k_fp8, int64_t k_seq_stride,
                           int64_t n_entries, const int32_t* pool_blocks, int32_t n_pool_blocks,
                           float* scores, float* block_max, hipStream_t stream) {
  const char* fn = "csa_index_score";
  ScoreArgs s{q_fp8, w, q_pos, n_seq, q_per_seq, k_fp8, k_seq_stride, n_entries, pool_blocks,
              n_pool_blocks, scores, block_max};
  if (n_seq * q_per_seq == 0 && n_seq >= 0 && q_per_seq >= 0) return CSA_OK;
  csa_status st = check_score(fn, s);
  if (st != CSA_OK) return st;
  return hip_status(launch_index_score(s, stream), fn);
}

// ------------------------------------------------------------------ a4 ----
size_t csa_topk_workspace_size(int64_t Q, int64_t ncols, int32_t k) {
  if (Q <= 0 || ncols <= 0 || k <= 0) return 0;
  return topk_workspace_bytes(Q, ncols, k);
}

csa_status csa_topk(const float* scores, int64_t Q, int64_t ncols, const int32_t* col_blocks, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "csa_topk";
  CHECK(Q >= 0, CSA_ERR_INVALID_ARG, "%s: Q < 0", fn);
  if (Q == 0) return CSA_OK;
  CHECK(ncols >= 1 && ncols < ((int64_t)1 << 31), CSA_ERR_UNSUPPORTED, "%s: ncols out of range", fn);
  CHECK(k >= 1 && k <= CSA_MAX_K, CSA_ERR_UNSUPPORTED, "%s: k must be in [1, 16384]", fn);
  CHECK(col_blocks == nullptr || ncols % 8 == 0, CSA_ERR_INVALID_ARG,
        "%s: pooled columns must be a multiple of 8", fn);
  CHECK_PTR(scores); CHECK_PTR(idx);
  CHECK_ALIGN(scores, 4); CHECK_ALIGN(idx, 4);
  if (col_blocks) CHECK_ALIGN(col_blocks, 4);
  size_t need = topk_workspace_bytes(Q, ncols, k);
  CHECK(need == 0 || (ws != nullptr && ws_bytes >= need), CSA_ERR_WORKSPACE,
        "%s: workspace needs %zu bytes", fn, need);
  if (need) CHECK_ALIGN(ws, 16);
  return hip_status(launch_topk(scores, Q, ncols, col_blocks, k, idx, ws, stream), fn);
}

// ------------------------------------------------------------------ a5 ----
size_t csa_block_pool_workspace_size(int64_t Q, int64_t ncols, int32_t is_block_max, int32_t nb) {
  if (Q <= 0 || ncols <= 0 || nb <= 0) return 0;
  return block_pool_workspace_bytes(Q, ncols, is_block_max, nb);
}

csa_status csa_block_pool(const float* values, int32_t is_block_max, int64_t Q, int64_t ncols,
                          int32_t n_pool_blocks, int32_t* pool_blocks, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  const char* fn = "csa_block_pool";
  CHECK(Q >= 0, CSA_ERR_INVALID_ARG, "%s: Q < 0", fn);
  if (Q == 0) return CSA_OK;
  CHECK(is_block_max == 0 || is_block_max == 1, CSA_ERR_INVALID_ARG, "%s: is_block_max must be 0 or 1", fn);
  CHECK(ncols >= 1 && ncols < ((int64_t)1 << 31), CSA_ERR_UNSUPPORTED, "%s: ncols out of range", fn);
  CHECK(n_pool_blocks >= 1 && n_pool_blocks <= 4096, CSA_ERR_UNSUPPORTED,
        "%s: n_pool_blocks must be in [1, 4096]", fn);
  CHECK_PTR(values); CHECK_PTR(pool_blocks);
  CHECK_ALIGN(values, 4); CHECK_ALIGN(pool_blocks, 4);
  size_t need = block_pool_workspace_bytes(Q, ncols, is_block_max, n_pool_blocks);
  CHECK(need == 0 || (ws != nullptr && ws_bytes >= need), CSA_ERR_WORKSPACE,
        "%s: workspace needs %zu bytes", fn, need);
  if (need) CHECK_ALIGN(ws, 256);
  return hip_status(launch_block_pool(values, is_block_max, Q, ncols, n_pool_blocks, pool_blocks, ws, stream),
                    fn);
}

// ------------------------------------------------------------------ a7 ----
size_t csa_sparse_attn_workspace_size(int64_t Q, int32_t k) {
  if (Q <= 0 || k <= 0) return 0;
  return attn_workspace_bytes(Q, k);
}

static csa_status check_attn(const char* fn, const float* q, const int32_t* q_pos, int64_t n_seq,
                             int64_t q_per_seq, const uint8_t* codes, const uint8_t* scales,
                             int64_t kv_rows, const int32_t* idx, int32_t k, const uint8_t* win,
                             int64_t win_cap, float sm_scale, float* out, void* ws, size_t ws_bytes) {
  CHECK(n_seq >= 0 && q_per_seq >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(k >= 1 && k <= CSA_MAX_K, CSA_ERR_UNSUPPORTED, "%s: k must be in [1, 16384]", fn);
  CHECK(kv_rows >= 0 && kv_rows < ((int64_t)1 << 23), CSA_ERR_UNSUPPORTED, "%s: kv_rows must be in [0, 2^23)", fn);
  CHECK(win_cap >= NWIN && win_cap < ((int64_t)1 << 22), CSA_ERR_UNSUPPORTED, "%s: win_cap must be in [128, 2^22)",
        fn);
  CHECK(std::isfinite(sm_scale), CSA_ERR_INVALID_ARG, "%s: sm_scale must be finite", fn);
  CHECK_PTR(q); CHECK_PTR(q_pos); CHECK_PTR(codes); CHECK_PTR(scales); CHECK_PTR(idx);
  CHECK_PTR(win); CHECK_PTR(out);
  CHECK_ALIGN(q, 16); CHECK_ALIGN(q_pos, 4); CHECK_ALIGN(codes, 16); CHECK_ALIGN(scales, 16);
  CHECK_ALIGN(idx, 4); CHECK_ALIGN(win, 16); CHECK_ALIGN(out, 16);
  size_t need = attn_workspace_bytes(n_seq * q_per_seq, k);
  CHECK(need == 0 || (ws != nullptr && ws_bytes >= need), CSA_ERR_WORKSPACE,
        "%s: workspace needs %zu bytes", fn, need);
  if (need) CHECK_ALIGN(ws, 16);
  return CSA_OK;
}

csa_status csa_sparse_attn(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                           const uint8_t* codes, const uint8_t* scales, int64_t kv_rows, const int32_t* idx,
                           int32_t k, const uint8_t* win, int64_t win_cap, float sm_scale, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "csa_sparse_attn";
  if (n_seq * q_per_seq == 0 && n_seq >= 0 && q_per_seq >= 0) return CSA_OK;
  csa_status st = check_attn(fn, q, q_pos, n_seq, q_per_seq, codes, scales, kv_rows, idx, k, win, win_cap,
                             sm_scale, out, ws, ws_bytes);
  if (st != CSA_OK) return st;
  return hip_status(launch_sparse_attn(q, q_pos, n_seq, q_per_seq, codes, scales, kv_rows, idx, k, win,
                                       win_cap, sm_scale, out, ws, stream),
                    fn);
}

// ----------------------------------------------- a7, allocation-free ----
// The split partials of csa_sparse_attn_noalloc live in this file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// must not pass the array's name to a kernel: its device address is looked
// up once per device with hipGetSymbolAddress and kept in g_scratch.
}  // extern "C"

static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, set on first use

// The current device's address of `scratch` (looked up with that device
// current, on the first call that needs it).
csa_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (p == nullptr) return fail(CSA_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CSA_OK;
}
}  // namespace

extern "C" {

size_t csa_noalloc_scratch_bytes(void) { return CSA_NOALLOC_SCRATCH_BYTES; }

csa_status csa_sparse_attn_noalloc(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                                   const uint8_t* codes, const uint8_t* scales, int64_t kv_rows,
                                   const int32_t* idx, int32_t k, const uint8_t* win, int64_t win_cap,
                                   float sm_scale, float* out, hipStream_t stream) {
  const char* fn = "csa_sparse_attn_noalloc";
  if (n_seq * q_per_seq == 0 && n_seq >= 0 && q_per_seq >= 0) return CSA_OK;
  CHECK(n_seq >= 0 && q_per_seq >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(k >= 1 && k <= CSA_MAX_K, CSA_ERR_UNSUPPORTED, "%s: k must be in [1, 16384]", fn);
  const size_t need = attn_workspace_bytes(n_seq * q_per_seq, k);
  CHECK(need <= CSA_NOALLOC_SCRATCH_BYTES, CSA_ERR_UNSUPPORTED,
        "%s: %lld queries at k = %d need %zu bytes of scratch; the static scratch holds %zu "
        "(use csa_sparse_attn with a workspace, or fewer queries per call)",
        fn, (long long)(n_seq * q_per_seq), k, need, (size_t)CSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    const csa_status st = scratch_address(fn, &ws);
    if (st != CSA_OK) return st;
  }
  csa_status st = check_attn(fn, q, q_pos, n_seq, q_per_seq, codes, scales, kv_rows, idx, k, win, win_cap,
                             sm_scale, out, ws, need);
  if (st != CSA_OK) return st;
  return hip_status(launch_sparse_attn(q, q_pos, n_seq, q_per_seq, codes, scales, kv_rows, idx, k, win,
                                       win_cap, sm_scale, out, ws, stream),
                    fn);
}

// ------------------------------------------------------------- a6 + a8 ----
size_t csa_layer_workspace_size(int32_t mode, const csa_layer_args* a) {
  if (a == nullptr || mode < CSA_MODE_FULL || mode > CSA_MODE_REUSE) return 0;
  return plan_layer(mode, a).total;
}

static csa_status check_layer(const char* fn, int32_t mode, const csa_layer_args* a, LayerPlan* plan) {
  CHECK(a != nullptr, CSA_ERR_INVALID_ARG, "%s: args is NULL", fn);
  CHECK(a->n_seq >= 0 && a->q_per_seq >= 0, CSA_ERR_INVALID_ARG, "%s: negative size", fn);
  CHECK(a->top_k >= 1 && a->top_k <= CSA_MAX_K, CSA_ERR_UNSUPPORTED, "%s: top_k must be in [1, 16384]", fn);
  CHECK(a->n_entries >= 0 && a->n_entries <= a->kv_rows, CSA_ERR_INVALID_ARG,
        "%s: n_entries must be <= kv_rows", fn);
  CHECK_PTR(a->idx); CHECK_PTR(a->out);
  if (mode != CSA_MODE_REUSE) {
    CHECK_PTR(a->q_idx); CHECK_PTR(a->w_idx); CHECK_PTR(a->k_fp8);
    CHECK(a->n_entries <= a->k_rows, CSA_ERR_INVALID_ARG, "%s: n_entries must be <= k_rows", fn);
    CHECK(a->n_entries >= 1, CSA_ERR_INVALID_ARG, "%s: n_entries must be >= 1", fn);
  }
  bool uses_pool = (mode == CSA_MODE_FULL && a->build_pool) || (mode == CSA_MODE_REINDEX && a->pool_blocks);
  if (mode == CSA_MODE_FULL && a->build_pool) CHECK_PTR(a->pool_blocks);
  if (uses_pool) {
    CHECK(a->n_pool_blocks >= 1 && a->n_pool_blocks <= 4096, CSA_ERR_UNSUPPORTED,
          "%s: n_pool_blocks must be in [1, 4096]", fn);
    CHECK_ALIGN(a->pool_blocks, 4);
  }
  if (mode == CSA_MODE_FULL && a->build_pool)
    CHECK(a->n_pool_blocks >= a->top_k, CSA_ERR_UNSUPPORTED,
          "%s: the pool must hold at least top_k blocks", fn);
  *plan = plan_layer(mode, a);
  CHECK(plan->total == 0 || (a->ws != nullptr && a->ws_bytes >= plan->total), CSA_ERR_WORKSPACE,
        "%s: workspace needs %zu bytes", fn, plan->total);
  if (plan->total) CHECK_ALIGN(a->ws, 256);
  if (mode != CSA_MODE_REUSE && plan->Q > 0) {
    ScoreArgs s{a->q_idx, a->w_idx, a->q_pos, a->n_seq, a->q_per_seq, a->k_fp8, a->k_rows, a->n_entries,
                plan->pooled ? a->pool_blocks : nullptr, a->n_pool_blocks, reinterpret_cast<float*>(256),
                nullptr};
    csa_status st = check_score(fn, s);
    if (st != CSA_OK) return st;
  }
  if (plan->Q > 0) {
    void* aws = reinterpret_cast<char*>(a->ws) + plan->off_attn;
    csa_status st = check_attn(fn, a->q_attn, a->q_pos, a->n_seq, a->q_per_seq, a->codes, a->scales,
                               a->kv_rows, a->idx, a->top_k, a->win, a->win_cap, a->sm_scale, a->out,
                               plan->total ? aws : nullptr, plan->total ? plan->total - plan->off_attn : 0);
    if (st != CSA_OK) return st;
  }
  return CSA_OK;
}

static csa_status run_attention(const char* fn, const csa_layer_args* a, const LayerPlan& p, hipStream_t st) {
  if (a->attn_after) {
    csa_status r = hip_status(hipStreamWaitEvent(st, a->attn_after, 0), fn);
    if (r != CSA_OK) return r;
  }
  void* aws = reinterpret_cast<char*>(a->ws) + p.off_attn;
  return hip_status(launch_sparse_attn(a->q_attn, a->q_pos, a->n_seq, a->q_per_seq, a->codes, a->scales,
                                       a->kv_rows, a->idx, a->top_k, a->win, a->win_cap, a->sm_scale,
                                       a->out, aws, st),
                    fn);
}

static csa_status run_index(const char* fn, int32_t mode, const csa_layer_args* a, const LayerPlan& p,
                            hipStream_t st) {
  char* ws = reinterpret_cast<char*>(a->ws);
  float* scores = (p.fused_full && !p.fused_scores) ? nullptr : reinterpret_cast<float*>(ws + p.off_scores);
  float* bm = (mode == CSA_MODE_FULL) ? reinterpret_cast<float*>(ws + p.off_bm) : nullptr;
  ScoreArgs s{a->q_idx, a->w_idx, a->q_pos, a->n_seq, a->q_per_seq, a->k_fp8, a->k_rows, a->n_entries,
              p.pooled ? a->pool_blocks : nullptr, a->n_pool_blocks, scores, bm};
  csa_status r = hip_status(launch_index_score(s, st), fn);
  if (r != CSA_OK) return r;
  if (mode != CSA_MODE_FULL)
    return hip_status(launch_topk(scores, p.Q, p.ncols, p.pooled ? a->pool_blocks : nullptr, a->top_k,
                                  a->idx, ws + p.off_sel, st),
                      fn);
  // Full: best blocks (the pool, or top_k blocks), then Top-K among their entries
  if (p.fused_full)
    return hip_status(launch_full_select(bm, p.nblk, p.Q, a->build_pool ? a->n_pool_blocks : a->top_k,
                                         a->build_pool ? a->pool_blocks : nullptr, a->top_k, a->idx, a->q_idx,
                                         a->w_idx, a->q_pos, a->q_per_seq, a->k_fp8, a->k_rows, a->n_entries,
                                         p.fused_scores ? scores : nullptr, p.split_full ? ws + p.off_split : nullptr,
                                         st),
                      fn);
  int32_t* blocks = a->build_pool ? a->pool_blocks : reinterpret_cast<int32_t*>(ws + p.off_blocks);
  const int32_t nb = a->build_pool ? a->n_pool_blocks : a->top_k;
  return hip_status(launch_pool_topk(bm, p.nblk, scores, p.ncols, p.Q, nb, blocks, a->top_k, a->idx,
                                    ws + p.off_sel, st),
                    fn);
}

csa_status csa_layer_full(const csa_layer_args* a, hipStream_t stream) {
  const char* fn = "csa_layer_full";
  LayerPlan p;
  csa_status st = check_layer(fn, CSA_MODE_FULL, a, &p);
  if (st != CSA_OK || p.Q == 0) return st;
  st = run_index(fn, CSA_MODE_FULL, a, p, stream);
  if (st != CSA_OK) return st;
  return run_attention(fn, a, p, stream);
}

csa_status csa_layer_reindex(const csa_layer_args* a, hipStream_t stream) {
  const char* fn = "csa_layer_reindex";
  LayerPlan p;
  csa_status st = check_layer(fn, CSA_MODE_REINDEX, a, &p);
  if (st != CSA_OK || p.Q == 0) return st;
  st = run_index(fn, CSA_MODE_REINDEX, a, p, stream);
  if (st != CSA_OK) return st;
  return run_attention(fn, a, p, stream);
}

csa_status csa_layer_reuse(const csa_layer_args* a, hipStream_t stream) {
  const char* fn = "csa_layer_reuse";
  LayerPlan p;
  csa_status st = check_layer(fn, CSA_MODE_REUSE, a, &p);
  if (st != CSA_OK || p.Q == 0) return st;
  return run_attention(fn, a, p, stream);
}

}  // extern "C"

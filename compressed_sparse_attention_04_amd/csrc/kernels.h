// Internal launchers of the libcsa kernels.  Arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// quant.hip
hipError_t launch_quantize(const float* e, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out,
                             hipStream_t st);
hipError_t launch_window_append(const float* x, int64_t n_seq, int64_t n_tok, int64_t x_seq_stride,
                                const int32_t* pos0, uint8_t* win, int64_t win_cap, hipStream_t st);
hipError_t launch_window_rebuild(const float* x, int64_t n_ring, int64_t n_tok, int64_t x_ring_stride,
                                 const int32_t* p_last, uint8_t* win, int64_t win_cap, hipStream_t st);
// A window append: token t of sequence s at x + s * x_seq_stride + t * 512
// goes to row (pos0[s] + t) % win_cap of ring s.
struct WindowAppendArgs {
  const float* x;
  int64_t n_seq, n_tok, x_seq_stride;
  const int32_t* pos0;
  uint8_t* win;
  int64_t win_cap;
};
size_t compress_workspace_bytes(int64_t n);
// append (optional): a window append done in the same launches
hipError_t launch_compress_quant(const float* x, int64_t n_seq, int64_t n_per_seq,
                                 int64_t x_seq_stride, const float* w, const float* rope_cs,
                                 int rope_dim, float eps, uint8_t* codes, uint8_t* scales,
                                 int64_t out_seq_stride, float* e_out, void* ws, hipStream_t st,
                                 const WindowAppendArgs* append = nullptr);

// index.hip
struct ScoreArgs {
  const uint8_t* q_fp8;   // [Q, 8, 128]
  const float* w;         // [Q, 8]
  const int32_t* q_pos;   // [Q]
  int64_t n_seq, q_per_seq;
  const uint8_t* k_fp8;   // [n_seq, k_rows, 128]
  int64_t k_rows;
  int64_t n_entries;
  const int32_t* pool;    // [Q, n_pool_blocks] or null
  int32_t n_pool_blocks;
  float* scores;          // [Q, ncols] or null
  float* block_max;       // [Q, ceil(ncols / 8)] or null
};
int64_t score_ncols(const ScoreArgs& a);
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t st);

// select.hip
size_t topk_workspace_bytes(int64_t Q, int64_t ncols, int32_t k);
hipError_t launch_topk(const float* scores, int64_t Q, int64_t ncols, const int32_t* col_blocks,
                       int32_t k, int32_t* idx, void* ws, hipStream_t st);
size_t topk_gather_workspace_bytes(int64_t Q, int64_t nmap, int32_t k);
hipError_t launch_topk_gather(const float* scores, int64_t Q, int64_t ncols, const int32_t* blocks,
                              int64_t nmap, int32_t k, int32_t* idx, void* ws, hipStream_t st);
size_t block_pool_workspace_bytes(int64_t Q, int64_t ncols, int32_t is_block_max, int32_t nb);
hipError_t launch_block_pool(const float* values, int32_t is_block_max, int64_t Q, int64_t ncols,
                             int32_t nb, int32_t* pool, void* ws, hipStream_t st);
// Full layer: the nb best blocks by block max -> pool [Q, nb], then the k best
// entries of those blocks -> idx [Q, k].  One kernel when a row fits one block.
size_t pool_topk_workspace_bytes(int64_t Q, int64_t nblk, int32_t nb, int32_t k);
hipError_t launch_pool_topk(const float* block_max, int64_t nblk, const float* scores, int64_t ncols,
                            int64_t Q, int32_t nb, int32_t* pool, int32_t k, int32_t* idx, void* ws,
                            hipStream_t st);

// full.hip: Full layer from block maxima alone (pool, then the Top-K of the
// rescored entries of the top_k blocks).
bool full_select_supported(int64_t nblk, int32_t nb, int32_t k);
// scores: the scan's scores [Q, n_entries] (decode batches: gathered for
// the chosen blocks), or null (their entries are rescored from k_fp8).
// split_ws (full_split_workspace_bytes, 256-byte aligned), or null: the
// rescoring and the Top-K run in a second kernel of several blocks per query.
hipError_t launch_full_select(const float* block_max, int64_t nblk, int64_t Q, int32_t nb, int32_t* pool,
                              int32_t k, int32_t* idx, const uint8_t* q_fp8, const float* w, const int32_t* q_pos,
                              int64_t q_per_seq, const uint8_t* k_fp8, int64_t k_rows, int64_t n_entries,
                              const float* scores, void* split_ws, hipStream_t st);
size_t full_split_top_bytes(int64_t Q, int32_t k);
size_t full_split_ticket_bytes(int64_t Q);
size_t full_split_workspace_bytes(int64_t Q, int32_t k);

// attn.hip
size_t attn_workspace_bytes(int64_t Q, int32_t k);
hipError_t launch_sparse_attn(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                              const uint8_t* codes, const uint8_t* scales, int64_t kv_rows,
                              const int32_t* idx, int32_t k, const uint8_t* win, int64_t win_cap,
                              float sm_scale, float* out, void* ws, hipStream_t st);

}  // namespace csa

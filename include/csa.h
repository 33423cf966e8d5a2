/*
 * csa.h -- C ABI of libcsa: one CSA2 compressed-sparse-attention layer step on
 * an AMD Instinct MI355X (gfx950).
 *
 * Sources of the method ("the pages"):
 *   "DeepSeek-V4.1 架构解析：把长上下文的成本瓶颈从算力挪到存储"
 *       (blog.yuzhonghai.cloud/deepseek-v41-arch), §02 CSA2 (layer modes
 *       Full / Reindex / Reuse, Top-512, the hierarchical pool of 2,048 blocks
 *       x 8 positions) and §03 精度与状态重建 (MXFP4 = E2M1 values with one E4M3
 *       scale per 16 channels, quantize after RoPE, FP4 for storage only, SWA
 *       KV in FP8, n_win = 128); cited below as "DeepSeek-V4.1 架构解析" §NN.
 *   The DeepSeek V4 overview page (wmrh.cn/news/159405) §2.1 (4:1
 *       compression of the predecessor).
 * The pages give no compressor or indexer formula and no dimensions; this
 * library implements the readings stated at each entry point.
 *
 * Conventions (every entry point):
 *   - Returns csa_status.  Arguments are validated on the host before any
 *     launch; on error nothing is enqueued and csa_last_error() (thread-local)
 *     describes the problem.
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     keeps none of them after returning and never allocates or frees device
 *     memory.  Scratch memory is a caller-provided workspace whose size the
 *     matching *_workspace_size function returns.
 *   - Work is enqueued asynchronously on the caller's stream; the library never
 *     synchronizes the device or the stream.
 *   - Rows of codes (256 B), scales (32 B), indexer keys (128 B) and window
 *     tokens (512 B) and every base pointer must be 16-byte aligned; float and
 *     int32 arrays must be 4-byte aligned (CSA_ERR_ALIGNMENT otherwise).
 *   - Every output element an entry point documents is written (including -1
 *     and -inf padding).
 *
 * Fixed dimensions (CSA_ERR_UNSUPPORTED for anything else):
 *   latent D = 512 (key = value), attention heads 16, indexer heads 8 x 128,
 *   tokens per entry 4, scale group 16, block 8, window 128 tokens.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_D 512
#define CSA_HEADS 16
#define CSA_IDX_HEADS 8
#define CSA_IDX_DIM 128
#define CSA_M 4
#define CSA_GROUP 16
#define CSA_CODE_BYTES 256   /* D / 2 */
#define CSA_SCALE_BYTES 32   /* D / 16 */
#define CSA_BLOCK 8
#define CSA_TOP_K 512
#define CSA_POOL_BLOCKS 2048
#define CSA_N_WIN 128
#define CSA_MAX_K 16384      /* largest k / top_k the selection and attention take */

typedef int32_t csa_status;
enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum value */
  CSA_ERR_UNSUPPORTED = 2, /* size outside what the kernels are built for */
  CSA_ERR_ALIGNMENT = 3,   /* pointer or row not aligned as required */
  CSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  CSA_ERR_HIP = 5,         /* a HIP launch failed; csa_last_error has the text */
  CSA_ERR_IO = 6           /* file open / read / write failed, or a file's header,
                              size or checksum is not what it must be */
};

/* Static text of a status code. */
const char* csa_status_string(csa_status s);
/* Text of the last error raised on the calling thread ("" if none). */
const char* csa_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int32_t csa_version(void);

/* ---------------------------------------------------------------- a2 ----
 * csa_quantize: MXFP4-quantize n post-RoPE entries ("DeepSeek-V4.1 架构解析" §03).
 *   e      [n, 512] float32, the quantizer input
 *   codes  [n, 256] uint8 out: channel 2k in the low nibble of byte k; each
 *          nibble = signbit(x) << 3 | RNE_E2M1(|x| / s) (saturating at 6,
 *          ties to the even code; magnitude 0 when s = 0)
 *   scales [n, 32] uint8 out: per 16-channel group s = RNE_E4M3FN(amax / 6),
 *          saturating at 448 (no global scale)
 * Decisions are exact: the result equals rounding the exact real quotients.
 * n = 0 is a no-op.
 */
csa_status csa_quantize(const float* e, int64_t n, uint8_t* codes, uint8_t* scales,
                        hipStream_t stream);

/* csa_dequantize: codes/scales of n entries -> float32 [n, 512] (s * E2M1(c)).
 * "DeepSeek-V4.1 架构解析" §03: the FP4 cache is dequantized before attention. */
csa_status csa_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n,
                          float* out, hipStream_t stream);

/* ----------------------------------------------------------- a1 + a2 ----
 * csa_compress_quant: compress every 4 token latents into one entry, RMSNorm,
 * RoPE, MXFP4-quantize and store ("DeepSeek-V4.1 架构解析" §02 sequence compression; the DeepSeek V4 overview page §2.1 4:1;
 * "DeepSeek-V4.1 架构解析" §03 RMSNorm magnitude ~1, quantize after RoPE).
 *   Entries are (sequence s < n_seq, r < n_per_seq).  Entry (s, r) reads the 4
 *   tokens x + s * x_seq_stride + r * 4 * 512 (float32 [4, 512]) and writes
 *   row s * out_seq_stride + r of codes [.., 256] / scales [.., 32].
 *   y = sum_i W_i x_i with w float32 [4, 512 (out), 512 (in)];
 *   e = y / sqrt(mean(y^2) + eps) (unit gain);
 *   RoPE on the last rope_dim channels (rope_dim even, 0 <= rope_dim <= 512,
 *   else CSA_ERR_UNSUPPORTED), pairs (c, c+1) rotated by rope_cs
 *   float32 [n_seq, n_per_seq, rope_dim / 2, 2] = (cos, sin); rope_cs may be
 *   NULL only when rope_dim = 0.
 *   e_out (optional, may be NULL): float32 [n_seq * n_per_seq, 512], the
 *   quantizer input (post-RoPE, float32), for inspection.
 *   Workspace: csa_compress_quant_workspace_size(n_seq * n_per_seq) bytes.
 */
size_t csa_compress_quant_workspace_size(int64_t n_entries);
csa_status csa_compress_quant(const float* x, int64_t n_seq, int64_t n_per_seq,
                              int64_t x_seq_stride, const float* w, const float* rope_cs,
                              int32_t rope_dim, float eps, uint8_t* codes, uint8_t* scales,
                              int64_t out_seq_stride, float* e_out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------- a9 ----
 * csa_window_append: write n_tok token latents of each of n_seq sequences into
 * the FP8 sliding-window ring ("DeepSeek-V4.1 架构解析" §03: SWA KV kept in FP8; n_win = 128).
 *   x       float32, token t of sequence s at x + s * x_seq_stride + t * 512
 *   pos0    int32 [n_seq]: position of token 0 of each sequence
 *   win     uint8 [n_seq, win_cap, 512]: token at position p goes to row
 *           p % win_cap; value = RNE_E4M3FN(x), saturating at +-448, sign kept
 *   win_cap >= 128 rows.
 */
csa_status csa_window_append(const float* x, int64_t n_seq, int64_t n_tok, int64_t x_seq_stride,
                             const int32_t* pos0, uint8_t* win, int64_t win_cap,
                             hipStream_t stream);

/* ------------------------------- compression and window append together ----
 * csa_compress_quant_append: csa_compress_quant and csa_window_append of the
 * same step in one call, for a decode or prefill step that completes entries
 * and appends its tokens: the two write different arrays, so the append's
 * threads run as extra blocks of the compression's second launch (two
 * launches instead of three).  The first fourteen arguments are those of
 * csa_compress_quant, the next seven (xw, nw_seq, nw_tok, xw_seq_stride,
 * pos0, win, win_cap) those of csa_window_append; either part may be empty
 * (n_seq * n_per_seq == 0 or nw_seq * nw_tok == 0), and an empty part's
 * arguments are not checked.  Results, validation and status codes are
 * those of the two calls; nothing is enqueued when either part is invalid.
 */
csa_status csa_compress_quant_append(const float* x, int64_t n_seq, int64_t n_per_seq, int64_t x_seq_stride,
                                     const float* w, const float* rope_cs, int32_t rope_dim, float eps,
                                     uint8_t* codes, uint8_t* scales, int64_t out_seq_stride, float* e_out,
                                     void* ws, size_t ws_bytes, const float* xw, int64_t nw_seq, int64_t nw_tok,
                                     int64_t xw_seq_stride, const int32_t* pos0, uint8_t* win, int64_t win_cap,
                                     hipStream_t stream);

/* ---------------------------------------------------------------- f2 ----
 * csa_window_rebuild: rebuild n_ring window rings from their latest tokens
 * ("DeepSeek-V4.1 架构解析" §03, SWA Bounded Replay: the window state is not kept in the
 * persistent cache; after a prefix-cache hit only the last n_win = 128
 * tokens are replayed).  One ring per (layer, sequence).
 *   x        float32: token i (0 <= i < n_tok) of ring r at
 *            x + r * x_ring_stride + i * 512; the last token (i = n_tok - 1)
 *            sits at position p_last[r] (>= 0), token i at
 *            p_last[r] - (n_tok - 1 - i)
 *   p_last   int32 [n_ring] (device)
 *   win      uint8 [n_ring, win_cap, 512] out (device), win_cap >= 128: row j
 *            of ring r gets RNE_E4M3FN (saturating, as csa_window_append) of
 *            the token at the latest position t <= p_last[r] with
 *            t = j (mod win_cap), when that token is among the n_tok given
 *            and t >= 0; every other row is zeroed.  With
 *            n_tok = min(128, p_last + 1) and win_cap = 128 the ring is
 *            byte-identical to appending every token of the history to a
 *            zeroed ring; with a larger win_cap the rows of the last 128
 *            positions are.
 *   1 <= n_tok <= win_cap; x_ring_stride a multiple of 4 and >= n_tok * 512
 *   when n_ring > 1; x, win 16-byte aligned.  The whole ring is written
 *   (no earlier contents are kept).
 */
csa_status csa_window_rebuild(const float* x, int64_t n_ring, int64_t n_tok, int64_t x_ring_stride,
                              const int32_t* p_last, uint8_t* win, int64_t win_cap,
                              hipStream_t stream);

/* ---------------------------------------------------------------- f4 ----
 * Global-KV files ("DeepSeek-V4.1 架构解析" §03: the global KV -- MXFP4 entries and indexer keys --
 * is what the persistent cache keeps; the window is rebuilt by replay).  One
 * file holds n_seq sequences' first n_entries rows of codes [.., 256], scales
 * [.., 32] and k_fp8 [.., 128], in device buffers laid out [n_seq, seq_rows,
 * row bytes].  Layout: a 64-byte header -- magic "CSA2GKV1", u32 version 1,
 * u32 header bytes 64, i64 n_seq, i64 n_entries, u32 row bytes 256 / 32 / 128,
 * u32 flags 0, u64 checksum, u64 reserved 0, little-endian -- then, for each
 * sequence, its code rows, scale rows and key rows.  The checksum is FNV-1a
 * over the payload read as little-endian 64-bit words (offset basis
 * 0xcbf29ce484222325, prime 0x100000001b3, one xor and one multiply per word).
 *
 * Unlike every other entry point, save and load block the calling thread
 * until the copies (on `stream`, after the work already queued there) and the
 * file I/O are done.  They copy through `stage`, a caller-provided host
 * buffer of stage_bytes >= 8 KiB, 16-byte aligned (pinned memory lets the
 * copies overlap the file I/O); the library allocates nothing.
 *
 * csa_kv_save: writes (or truncates and rewrites) `path`.  0 <= n_entries <=
 *   seq_rows.  CSA_ERR_IO if the file cannot be created or written.
 * csa_kv_load: reads a file written by csa_kv_save into the buffers; the file
 *   must hold n_seq sequences and at most seq_rows entries each
 *   (CSA_ERR_INVALID_ARG otherwise, nothing copied); *n_entries_out = the
 *   file's n_entries; rows past it are left as they are.  CSA_ERR_IO for a
 *   bad header, a size that does not match it, a read error, or a checksum
 *   mismatch -- in the last case the buffers already hold the file's
 *   (damaged) rows.
 * csa_kv_file_info: host only; checks the header and the file size and
 *   returns the file's n_seq and n_entries (CSA_ERR_IO as above, checksum
 *   not verified).
 */
csa_status csa_kv_save(const char* path, const uint8_t* codes, const uint8_t* scales, const uint8_t* k_fp8,
                       int64_t n_seq, int64_t seq_rows, int64_t n_entries, void* stage, size_t stage_bytes,
                       hipStream_t stream);
csa_status csa_kv_load(const char* path, uint8_t* codes, uint8_t* scales, uint8_t* k_fp8, int64_t n_seq,
                       int64_t seq_rows, int64_t* n_entries_out, void* stage, size_t stage_bytes,
                       hipStream_t stream);
csa_status csa_kv_file_info(const char* path, int64_t* n_seq, int64_t* n_entries);

/* -------------------------------------------------------- measurement ----
 * Probes of what the GPU sustains for the indexer's two resources (not part
 * of the method; the benchmark reports the indexer against them beside the
 * published peaks).
 * csa_probe_mfma_f16: `blocks` blocks of 256 threads, every wave running
 *   iters x 32 independent v_mfma_f32_16x16x32_f16 (16,384 multiply-adds
 *   each); out: one float (device), written only to keep the work live.
 * csa_probe_mfma_f8: as csa_probe_mfma_f16 for the FP8 matrix instructions:
 *   variant 0 = v_mfma_scale_f32_16x16x128_f8f6f4 on E4M3 operands (65,536
 *   flops each), variant 1 = v_mfma_f32_16x16x32_fp8_fp8 (16,384 flops).
 * csa_probe_read: reads `bytes` (a multiple of 16, buf 16-byte aligned) with
 *   whole-line non-temporal 16-byte loads; out as above.
 */
csa_status csa_probe_mfma_f16(float* out, int32_t blocks, int32_t iters, hipStream_t stream);
csa_status csa_probe_mfma_f8(float* out, int32_t blocks, int32_t iters, int32_t variant, hipStream_t stream);
csa_status csa_probe_read(const uint8_t* buf, int64_t bytes, float* out, hipStream_t stream);

/* ---------------------------------------------------------------- a3 ----
 * csa_index_score: indexer scores of Q = n_seq * q_per_seq queries ("DeepSeek-V4.1 架构解析" §02:
 * Full layers score every causally visible position; Reindex layers rescore
 * with their own query, inside the hierarchical pool when one exists).
 *   Query q belongs to sequence q / q_per_seq and sits at token position
 *   q_pos[q] >= 0; entry j is visible iff 4j + 3 <= q_pos[q].
 *   score = sum_h w[q, h] * ReLU(q_fp8[q, h, :] . k_fp8[j, :]) (8 heads x 128,
 *   E4M3 operands; every dot product is exact before its one float32
 *   rounding, as the operands are widened to fp16 for the matrix cores).
 *   q_fp8 uint8 [Q, 8, 128]; w float32 [Q, 8] (must be >= 0);
 *   k_fp8 uint8 [n_seq, k_seq_stride, 128].
 *   Dense mode (pool_blocks == NULL): ncols = n_entries columns; column j is
 *   entry j (j < n_entries <= k_seq_stride).
 *   Pooled mode: pool_blocks int32 [Q, n_pool_blocks] (ascending block ids,
 *   -1 padded); ncols = 8 * n_pool_blocks; column c is entry
 *   8 * pool[c / 8] + c % 8.
 *   scores (may be NULL) float32 [Q, ncols] out; invisible columns, entries
 *   >= n_entries and -1 pool slots are written as -inf.
 *   block_max (may be NULL; dense mode only) float32 [Q, ceil(ncols / 8)] out:
 *   max score of each aligned 8-entry block over its visible entries (-inf if
 *   none).  At least one of scores / block_max must be given.
 */
csa_status csa_index_score(const uint8_t* q_fp8, const float* w, const int32_t* q_pos,
                           int64_t n_seq, int64_t q_per_seq, const uint8_t* k_fp8,
                           int64_t k_seq_stride, int64_t n_entries, const int32_t* pool_blocks,
                           int32_t n_pool_blocks, float* scores, float* block_max,
                           hipStream_t stream);

/* ---------------------------------------------------------------- a4 ----
 * csa_topk: for each of Q rows of scores float32 [Q, ncols], select the k
 * columns with the largest scores ("DeepSeek-V4.1 架构解析" §02 Top-512); equal scores go to the
 * lower column (-0 equals +0); -inf and NaN columns are never selected.
 * Outputs the selected ids in
 * ascending order, -1 padded, into idx int32 [Q, k].
 *   col_blocks (may be NULL) int32 [Q, ncols / 8]: when given, column c maps
 *   to id 8 * col_blocks[q, c / 8] + c % 8 (pooled scores; the block ids must
 *   be ascending so that id order equals column order).
 *   1 <= k <= 16384 (CSA_MAX_K); ncols >= 1.  A k at or above the number of
 *   valid columns selects every valid column (the dense case).
 *   Workspace: csa_topk_workspace_size(Q, ncols, k).
 */
size_t csa_topk_workspace_size(int64_t Q, int64_t ncols, int32_t k);
csa_status csa_topk(const float* scores, int64_t Q, int64_t ncols, const int32_t* col_blocks,
                    int32_t k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- a5 ----
 * csa_block_pool: the hierarchical pool ("DeepSeek-V4.1 架构解析" §02: rank 8-position blocks by
 * their largest index score, keep 2,048 blocks = 16,384 candidates).
 *   is_block_max = 1: values float32 [Q, ncols] are block maxima (one column
 *   per block); 0: values are per-entry scores and the block maxima over
 *   aligned 8-column blocks are formed first (-inf entries ignored).
 *   Selects n_pool_blocks blocks per row by (block max desc, block id asc),
 *   -inf blocks never; writes ascending block ids, -1 padded, to
 *   pool_blocks int32 [Q, n_pool_blocks].  1 <= n_pool_blocks <= 4096.
 *   Workspace: csa_block_pool_workspace_size(Q, ncols, is_block_max, n_pool_blocks).
 */
size_t csa_block_pool_workspace_size(int64_t Q, int64_t ncols, int32_t is_block_max,
                                     int32_t n_pool_blocks);
csa_status csa_block_pool(const float* values, int32_t is_block_max, int64_t Q, int64_t ncols,
                          int32_t n_pool_blocks, int32_t* pool_blocks, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------- a7 ----
 * csa_sparse_attn: sparse multi-query attention ("DeepSeek-V4.1 架构解析" §02 the selected entries
 * are used for attention; "DeepSeek-V4.1 架构解析" §03 the FP4 cache is dequantized before
 * attention and the SWA window stays FP8, n_win = 128).
 *   Query q (sequence q / q_per_seq, position q_pos[q]) attends with 16 heads
 *   q float32 [Q, 16, 512] over the union of
 *     - the entries idx int32 [Q, k] (ids < 0 or >= kv_rows are skipped),
 *       dequantized from codes [n_seq, kv_rows, 256] / scales [n_seq, kv_rows, 32]
 *       (one shared latent is both key and value), and
 *     - the window tokens max(0, p - 127) .. p, read from
 *       win uint8 [n_seq, win_cap, 512] row p % win_cap (E4M3, no scale),
 *   with one softmax of logits sm_scale * q . key.  out float32 [Q, 16, 512].
 *   Arithmetic: keys and values are exact in fp16; q and the softmax weights
 *   are each carried as two fp16 halves (hi + lo, ~2^-22 relative) on the
 *   fp16 matrix cores with float32 accumulation; float32 softmax.
 *   1 <= k <= 16384 (CSA_MAX_K); kv_rows < 2^23 (8,388,608 entries, a
 *   33.5M-token context); 128 <= win_cap < 2^22 (CSA_ERR_UNSUPPORTED otherwise).
 *   Workspace: csa_sparse_attn_workspace_size(Q, k).
 */
size_t csa_sparse_attn_workspace_size(int64_t Q, int32_t k);
csa_status csa_sparse_attn(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                           const uint8_t* codes, const uint8_t* scales, int64_t kv_rows,
                           const int32_t* idx, int32_t k, const uint8_t* win, int64_t win_cap,
                           float sm_scale, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* --------------------------------------------------- a7, no allocation ----
 * csa_sparse_attn_noalloc: csa_sparse_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same arguments and result, without a
 * workspace.  The split partials go to a static device scratch of
 * CSA_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends; this call allocates and frees nothing.
 *   The call runs on the current device; csa_sparse_attn_workspace_size(Q, k)
 *   must not exceed the scratch (about 199 decode queries at k = 512;
 *   prefill plans of 512+ queries need none), else CSA_ERR_UNSUPPORTED and
 *   nothing is enqueued.  The scratch holds no state between calls (every
 *   partial is written before it is read).  All calls on one GPU share the
 *   one scratch: calls that overlap in time on that GPU (on different
 *   streams, or from different threads) race and must be ordered by the
 *   caller.
 * csa_noalloc_scratch_bytes: CSA_NOALLOC_SCRATCH_BYTES.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
size_t csa_noalloc_scratch_bytes(void);
csa_status csa_sparse_attn_noalloc(const float* q, const int32_t* q_pos, int64_t n_seq, int64_t q_per_seq,
                                   const uint8_t* codes, const uint8_t* scales, int64_t kv_rows,
                                   const int32_t* idx, int32_t k, const uint8_t* win, int64_t win_cap,
                                   float sm_scale, float* out, hipStream_t stream);

/* ------------------------------------------------------------ a6 + a8 ----
 * Layer entry points ("DeepSeek-V4.1 架构解析" §02 layer modes).
 *   Full:    score every visible entry with (q_idx, w_idx) -> Top-k idx;
 *            when build_pool != 0 also the hierarchical pool -> pool_blocks.
 *   Reindex: reuse the Full layer's cache, indexer keys and pool; rescore
 *            inside the pool (or every visible entry if pool_blocks is NULL)
 *            with this layer's (q_idx, w_idx) -> Top-k idx.
 *   Reuse:   attention with the idx given (the most recent Full/Reindex).
 *   All three then run csa_sparse_attn with q_attn -> out.
 * Field meanings follow the entry points above.  Workspace:
 *   csa_layer_workspace_size(mode, args) with mode CSA_MODE_*.
 * attn_after (optional, NULL for none): an event the layer's attention waits
 *   for on `stream` (hipStreamWaitEvent) before it starts; the scoring and
 *   selection do not wait.  A step uses it to compress and store its new
 *   entries on a second stream while the Full layer scores and selects, since
 *   only the attention reads the cache rows and window that the compression
 *   writes ("DeepSeek-V4.1 架构解析" §02, §03).  The event is not owned by the
 *   library; an error from the wait is returned as CSA_ERR_HIP.
 */
enum { CSA_MODE_FULL = 0, CSA_MODE_REINDEX = 1, CSA_MODE_REUSE = 2 };

typedef struct csa_layer_args {
  /* cache view (per sequence: kv_rows rows) */
  const uint8_t* codes;    /* [n_seq, kv_rows, 256] */
  const uint8_t* scales;   /* [n_seq, kv_rows, 32] */
  int64_t kv_rows;
  const uint8_t* k_fp8;    /* [n_seq, k_rows, 128] */
  int64_t k_rows;
  int64_t n_entries;       /* entries in use per sequence (<= kv_rows, k_rows) */
  const uint8_t* win;      /* [n_seq, win_cap, 512] */
  int64_t win_cap;
  /* queries */
  int64_t n_seq;
  int64_t q_per_seq;
  const int32_t* q_pos;    /* [Q] */
  const float* q_attn;     /* [Q, 16, 512] */
  const uint8_t* q_idx;    /* [Q, 8, 128] (Full, Reindex) */
  const float* w_idx;      /* [Q, 8] (Full, Reindex) */
  float sm_scale;
  int32_t top_k;           /* k (512 for the method), 1 .. 16384, and at most
                              n_pool_blocks with build_pool */
  int32_t build_pool;      /* Full: also build the pool */
  int32_t n_pool_blocks;   /* 2048 for the method */
  int32_t* pool_blocks;    /* [Q, n_pool_blocks]: out (Full + build_pool), in (Reindex) */
  int32_t* idx;            /* [Q, top_k]: out (Full, Reindex), in (Reuse) */
  float* out;              /* [Q, 16, 512] */
  void* ws;
  size_t ws_bytes;
  hipEvent_t attn_after;   /* optional: the attention waits for this event */
} csa_layer_args;

size_t csa_layer_workspace_size(int32_t mode, const csa_layer_args* a);
csa_status csa_layer_full(const csa_layer_args* a, hipStream_t stream);
csa_status csa_layer_reindex(const csa_layer_args* a, hipStream_t stream);
csa_status csa_layer_reuse(const csa_layer_args* a, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */

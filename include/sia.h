/*
 * libsia — sparse index attention on AMD Instinct MI355X (gfx950).
 *
 * The path: a lightweight indexer scores every causal history position of each
 * query token, a per-query Top-K keeps the K best positions, and a sparse
 * attention kernel over a paged low-rank (MLA) latent KV cache reads only those
 * K rows.
 *
 * Pages cited (Baidu AI Cloud articles):
 *   [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models"
 *   [P2] "Efficient Inference Deployment and Optimization for Hybrid Attention LLMs"
 *   [P3] "Day-One Inference Adaptation for Very Large Hybrid-Attention Models:
 *         From Operators to Serving Systems"
 *   [P4] "Inference Acceleration for New LLM Architectures: Day-0 Adaptation and
 *         Sparse Attention Optimization"
 *   [P5] "Inference Adaptation and Performance Optimization for a Domestically
 *         Developed LLM's New Architecture"
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory), row-major with
 *     the last dimension contiguous, owned by the caller.  The library never
 *     allocates, frees or keeps a pointer after returning.  (The one device
 *     array it holds is the workspace of sia_index_select_attend_noalloc.)
 *   - Work is enqueued asynchronously on `stream`; nothing synchronizes the host.
 *     The caller synchronizes before reading outputs.
 *   - Arguments are validated on the host before anything is launched.  On a
 *     validation failure the call returns a negative sia_status and leaves every
 *     output untouched.  A failed launch returns SIA_ERR_HIP.
 *   - Device-resident metadata (q_pos, q_seq, block tables, indices) cannot be
 *     checked on the host.  The kernels clamp it so that no access leaves its
 *     buffer, but values outside the documented ranges give unspecified results.
 *   - Calls are thread-safe.  The only global state is the per-GPU address of
 *     the sia_index_select_attend_noalloc workspace, looked up under a lock.
 *   - fp8 is OCP e4m3fn (bias 7, max 448, no infinities), gfx950's native format.
 *   - Dequantization scales must be finite and > 0.
 */
#ifndef SIA_H
#define SIA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SIA_OK = 0,
  SIA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, bad range */
  SIA_ERR_UNSUPPORTED = -2, /* well-formed but outside the supported shapes/dtypes */
  SIA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than sia_workspace_size */
  SIA_ERR_HIP = -4          /* a HIP launch failed */
} sia_status;

typedef enum { SIA_F32 = 0, SIA_BF16 = 1, SIA_FP8_E4M3 = 2, SIA_MXFP8_E4M3 = 3 } sia_dtype;

/* Query -> sequence map shared by every step.  Varlen batches are described by
 * vectors of offsets instead of per-sequence loops [P3, section 3.1].
 *   q_seq[T]          sequence id of query row t, in [0, batch)
 *   q_pos[T]          logical position of query t; keys 0..q_pos[t] are visible
 *                     (causal history, diagonal included [P1, "Prefill Context
 *                     Parallelism"]).  Must be < max_visible and < the sequence's
 *                     length in the cache.
 *   block_table[batch, max_pages]  physical page of each logical page; logical
 *                     position s of sequence b lives in slot
 *                     block_table[b][s / page_size] * page_size + s % page_size
 *                     of every pool (indexer keys and latent KV share it).
 *   num_tokens        T (>= 0; T = 0 is a no-op)
 *   batch             number of sequences (>= 1)
 *   page_size         tokens per page; must be 64
 *   num_pages         pages in each pool; page ids are clamped to it
 *   max_visible       host-side bound: q_pos[t] + 1 <= max_visible for all t;
 *                     must be <= max_pages * page_size                        */
typedef struct {
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* block_table;
  int32_t num_tokens;
  int32_t batch;
  int32_t max_pages;
  int32_t page_size;
  int32_t num_pages;
  int32_t max_visible;
} sia_seqmap;

/* Indexer inputs [P1, "Sparse Attention Pipeline Optimization"; P2, section 3.1].
 *   q        [T, heads, dim]  e4m3 codes (SIA_FP8_E4M3, SIA_MXFP8_E4M3),
 *            bfloat16 (SIA_BF16: the precision path, no scales [P2, section
 *            3.2; P5, section 3.1]) or float (SIA_F32); with q_bf16 = 1, bfloat16 queries that are
 *            quantized on the fly to the indexer's format (see
 *            sia_quantize_indexer_q); q_scale is then unused
 *   q_scale  SIA_FP8_E4M3: float [T] (q_scale_per_head = 0) or [T, heads] (= 1)
 *            SIA_MXFP8_E4M3: uint8 [T, heads, dim/32], one OCP E8M0 scale
 *            (2^(e-127)) per 32 consecutive elements of a head's q [P1,
 *            "Hierarchical Quantization"; P2, section 4.1]; 4-byte aligned
 *   w        [T, heads] float head weights
 *   k_pool   [num_pages, page_size, dim] keys, same dtype as q; one key vector
 *            per token shared by all indexer heads
 *   k_scale  SIA_FP8_E4M3: float [num_pages, page_size], one per key token
 *            SIA_MXFP8_E4M3: uint8 [num_pages, page_size, dim/32] E8M0 group
 *            scales; 4-byte aligned
 * Supported: SIA_F32 with heads <= 64, dim <= 256; SIA_BF16, SIA_FP8_E4M3 and
 * SIA_MXFP8_E4M3 with heads in {32, 64} and dim = 128.                        */
typedef struct {
  const void* q;
  const void* q_scale;
  const float* w;
  const void* k_pool;
  const void* k_scale;
  sia_dtype dtype;
  int32_t q_scale_per_head;
  int32_t heads;
  int32_t dim;
  int32_t q_bf16;  /* 1: q holds bfloat16 values to quantize (fp8 / MXFP8 indexers only) */
} sia_indexer_in;

/* Latent KV cache [P1, "Hierarchical Quantization"; P5, section 4 table].
 *   kv_pool  SIA_BF16: [num_pages, page_size, latent+rope] bfloat16
 *            SIA_F32 : [num_pages, page_size, latent+rope] float
 *            SIA_FP8_E4M3: [num_pages, page_size, latent + 2*rope] bytes per row:
 *                      latent e4m3 codes, then rope as bfloat16
 *   kv_scale fp8 only: one float per tile of scale_tokens consecutive tokens of
 *            a page and scale_elems consecutive latent elements, laid out
 *            [num_pages, page_size/scale_tokens, latent/scale_elems].
 *            Supported tiles: (64, 512) one scale per page, (1, 128) per token
 *            and 128-element tile.
 * Supported: SIA_F32 with latent+rope <= 1024; SIA_BF16 / SIA_FP8_E4M3 with
 * latent = 512, rope = 64.                                                     */
typedef struct {
  const void* kv_pool;
  const float* kv_scale;
  sia_dtype dtype;
  int32_t scale_tokens;
  int32_t scale_elems;
  int32_t latent_dim;
  int32_t rope_dim;
} sia_kv_in;

/* Operation codes for sia_workspace_size. */
enum { SIA_OP_TOPK = 0, SIA_OP_MLA_DECODE = 1, SIA_OP_MLA_PREFILL = 2, SIA_OP_INDEX_SELECT_ATTEND = 3,
       SIA_OP_INDEX_TOPK = 4, SIA_OP_TOPK_PAGES = 5 };

/* Values of the `order` argument of the selecting calls.
 *   SIA_ORDER_SCORE     per-position Top-K, written best first
 *   SIA_ORDER_POSITION  the same set, written in ascending position
 *   SIA_SELECT_PAGES    block-aligned selection (sia_topk_pages): whole pages
 *                       of the cache, positions written in ascending order;
 *                       K must be a multiple of the page size (64)           */
enum { SIA_ORDER_SCORE = 0, SIA_ORDER_POSITION = 1, SIA_SELECT_PAGES = 2 };

/* Step 1 — indexer scores [P1, "Sparse Attention Pipeline Optimization";
 * P2, section 3.1; P3, section 3.1].
 *   scores[t * ld + s] = sum_h w[t,h] * ReLU(qs[t,h] * ks[s] * <q[t,h], k[s]>)
 * for s = 0..q_pos[t] (fp32 accumulate).  Entries s > q_pos[t] are not part of
 * the result: entries q_pos[t] < s < max_visible may be overwritten with -inf,
 * entries s >= max_visible are never written.
 *   scores  [T, ld] float, 16-byte aligned; ld % 4 == 0, ld >= max_visible.     */
int sia_index_scores(const sia_indexer_in* in, const sia_seqmap* seq, float* scores,
                     int64_t ld, hipStream_t stream);

/* Step 2 — per-query Top-K [P1, "Sparse Attention Pipeline Optimization";
 * P2, section 3.2].  For each row t, over candidates s = 0..q_pos[t] of
 * scores[t * ld + s], keeps the first min(K, q_pos[t] + 1) positions under the
 * order (score descending, position ascending), -0.0 equal to +0.0, and pads
 * idx with -1 up to K.  order = 0 writes them in that order; order = 1 writes
 * the same set in ascending position.  Scores must be finite.
 *   idx   [T, K] int32 logical positions (the index representation shared with
 *         the cache layer [P3, section 4])
 *   vals  [T, K] float or NULL: the selected scores (-inf for padding)
 * Supported: 1 <= K <= 2048.  No workspace.                                     */
int sia_topk(const float* scores, int64_t ld, const sia_seqmap* seq, int32_t K, int32_t order,
             int32_t* idx, float* vals, hipStream_t stream);

/* Step 2, block-aligned form [P3, section 3.1: the selection is aligned to
 * cache blocks so that attention reads the cache block by block].  The page
 * leaves the block ranking open; here a page (64 consecutive positions, the
 * cache block) scores the largest of scores[t * ld + s] over its positions
 * s <= q_pos[t].  Keeps the first min(K / 64, pages) pages under (page score
 * descending, page ascending), -0.0 equal to +0.0, and writes every visible
 * position of the kept pages in ascending order, then -1 up to K (so the -1
 * entries trail).  Rows with q_pos[t] + 1 <= K keep every visible position.
 * Scores must be finite.
 *   idx   [T, K] int32 logical positions
 *   vals  [T, K] float or NULL: each position's page score (-inf for padding)
 *   ws    at least sia_workspace_size(SIA_OP_TOPK_PAGES, ...) bytes, 256-byte
 *         aligned (page scores and the kept pages)
 * Supported: K a multiple of 64, 64 <= K <= 2048 (else SIA_ERR_INVALID_ARG /
 * SIA_ERR_UNSUPPORTED).                                                        */
int sia_topk_pages(const float* scores, int64_t ld, const sia_seqmap* seq, int32_t K, int32_t* idx,
                   float* vals, void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps 1 + 2 fused — indexer scores and per-query Top-K without a score
 * matrix in memory [P1, "Sparse Attention Pipeline Optimization" (indexer
 * fusion); P4, section 2; P5, section 3.1].  Same result as sia_index_scores
 * followed by sia_topk on those scores (same arguments and conventions as
 * sia_topk for K, order, idx and vals), whichever method runs:
 *   SIA_INDEX_TOPK_ONCHIP  (fp8 and MXFP8 indexers) each range of 8192 keys of a
 *       query is scored into on-chip memory and reduced to its own best
 *       min(K, keys) entries, which go to the workspace; a second pass selects
 *       the query's Top-K from them.  One workgroup per (query, range): suits
 *       decode-like batches, where every query has its own keys.
 *   SIA_INDEX_TOPK_SCORES  scores go through a matrix in the workspace
 *       (sia_index_scores, then sia_topk).
 *   SIA_INDEX_TOPK_AUTO    the on-chip method for fp8 and MXFP8 indexers when there are
 *       at most two queries per sequence on average and at least one
 *       (query, range) pair per compute unit; the score matrix otherwise.
 * order = SIA_SELECT_PAGES gives sia_topk_pages' block-aligned selection (the
 * score-matrix method; SIA_INDEX_TOPK_ONCHIP is then SIA_ERR_UNSUPPORTED).
 *   ws  workspace of at least sia_workspace_size(SIA_OP_INDEX_TOPK, ...) bytes
 *       (enough for either method), 256-byte aligned; heads and latent_dim
 *       are ignored for this op.
 * Errors: SIA_ERR_UNSUPPORTED for SIA_INDEX_TOPK_ONCHIP with an fp32 indexer. */
enum { SIA_INDEX_TOPK_AUTO = 0, SIA_INDEX_TOPK_ONCHIP = 1, SIA_INDEX_TOPK_SCORES = 2 };
int sia_index_topk(const sia_indexer_in* in, const sia_seqmap* seq, int32_t K, int32_t order, int32_t method,
                   int32_t* idx, float* vals, void* ws, size_t ws_bytes, hipStream_t stream);
/* The method SIA_INDEX_TOPK_AUTO picks for these arguments (host-side only; a
 * negative status for arguments sia_index_topk would reject).                 */
int sia_index_topk_method(const sia_indexer_in* in, const sia_seqmap* seq);

/* Dynamic Q quantization — the weight-free step of the indexer prolog [P2,
 * section 3.2 (Q quantization on the decode critical path); P2, section 4.1 and
 * P5, section 4 table (MXFP8 groups of 32)].  in->q holds bfloat16 queries
 * [T, heads, dim] (in->q_bf16 = 1); the result is what sia_index_scores takes
 * for in->dtype:
 *   SIA_FP8_E4M3: q_codes [T, heads, dim] e4m3, q_scales float [T]:
 *       scale = amax / 448 over the token, codes = e4m3(x * (448 / amax))
 *       (fp32, round to nearest even; a token of zeros: scale 1, zero codes)
 *   SIA_MXFP8_E4M3: q_codes as above, q_scales uint8 [T, heads, dim/32]: per
 *       32 elements the smallest 2^e with amax <= 448 * 2^e (E8M0 byte e+127,
 *       0 for an all-zero group), codes = e4m3(x * 2^-e)
 * e4m3 rounding is to the nearest value, ties to the even code, saturating at
 * 448.  q_codes 16-byte aligned, q_scales 4-byte aligned.  sia_index_topk and
 * sia_index_select_attend run this step themselves (into their workspace) when
 * in->q_bf16 = 1; sia_index_scores requires quantized input (else
 * SIA_ERR_UNSUPPORTED).                                                       */
int sia_quantize_indexer_q(const sia_indexer_in* in, int32_t num_tokens, void* q_codes, void* q_scales,
                           hipStream_t stream);

/* Step 3 — sparse MLA attention over the selected rows [P1, "Sparse Attention
 * Pipeline Optimization"; P3, section 3.2].  For each token t and head h, over
 * the rows j = idx[t, i] != -1 (logical positions of sequence q_seq[t]):
 *   l_j = softmax_scale * <q[t,h,:], kv_j[0:latent+rope]>
 *   out[t,h,:] = sum_j softmax(l)_j * kv_j[0:latent],   lse[t,h] = log sum_j e^l_j
 * The key is the whole latent+rope row, the value its latent part, shared by
 * all heads.  A token with no valid index gets out = 0 and lse = -inf.
 *   q     [T, heads, latent+rope]: SIA_BF16 for bf16/fp8 caches, SIA_F32 for f32
 *   out   [T, heads, latent] in q's dtype;  lse [T, heads] float or NULL
 *   idx   [T, K] int32 (-1 = unused slot; an unused slot, or a position
 *         outside [0, max_visible), reads nothing from the pools and
 *         contributes nothing, whatever the pool holds)
 * Supported: f32 cache with heads <= 64; bf16/fp8 cache with heads in
 * {32, 64, 128}.  1 <= K <= 2048.
 * _decode splits each token's rows over several workgroups and merges the
 * partial results in a fixed order (needs workspace, see sia_workspace_size);
 * _prefill gives each token one workgroup (no workspace; ws may be NULL).      */
int sia_sparse_mla_decode(const void* q, sia_dtype q_dtype, int32_t heads, const sia_kv_in* kv,
                          const sia_seqmap* seq, const int32_t* idx, int32_t K,
                          float softmax_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                          hipStream_t stream);
int sia_sparse_mla_prefill(const void* q, sia_dtype q_dtype, int32_t heads, const sia_kv_in* kv,
                           const sia_seqmap* seq, const int32_t* idx, int32_t K,
                           float softmax_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* The whole path in one call: scores -> Top-K -> sparse MLA [P1, "Sparse
 * Attention Pipeline Optimization" pseudo-code; P4, section 2].  Steps 1 + 2
 * run as sia_index_topk with SIA_INDEX_TOPK_AUTO; its scratch and (when
 * idx_out is NULL) the indices live in the workspace.  Uses the split
 * (decode) attention when there are too few tokens to fill the GPU.
 *   idx_out [T, K] int32 or NULL; `order` as in sia_topk, or SIA_SELECT_PAGES
 *           for the block-aligned selection of sia_topk_pages.                */
int sia_index_select_attend(const sia_indexer_in* in, const void* q_mla, sia_dtype q_dtype,
                            int32_t heads, const sia_kv_in* kv, const sia_seqmap* seq, int32_t K,
                            int32_t order, float softmax_scale, int32_t* idx_out, void* out,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole path in one call without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments and results are those of
 * sia_index_select_attend.  The workspace is a device array inside the
 * library, SIA_NOALLOC_WORKSPACE_BYTES per GPU, allocated when the library's
 * code is loaded on that GPU and held until the process ends; the call itself
 * allocates nothing.  A call whose sia_workspace_size(SIA_OP_INDEX_SELECT_ATTEND,
 * ...) exceeds that size returns SIA_ERR_WORKSPACE before anything is
 * launched (decode batches fit: 64 sequences x 32768 tokens need 41.2 MiB;
 * long prefills, whose score matrix is T x max_visible floats, do not).  Every
 * call on one GPU uses that GPU's array: calls that may overlap on one GPU
 * (different streams without ordering between them) race and must be
 * serialized by the caller.  Nothing in the array needs to start cleared.     */
#define SIA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int sia_index_select_attend_noalloc(const sia_indexer_in* in, const void* q_mla, sia_dtype q_dtype,
                                    int32_t heads, const sia_kv_in* kv, const sia_seqmap* seq, int32_t K,
                                    int32_t order, float softmax_scale, int32_t* idx_out, void* out,
                                    float* lse, hipStream_t stream);

/* Bytes of workspace `op` needs for this sequence map, K, heads and latent
 * dimension (0 when none).  Returns (size_t)-1 for invalid arguments.          */
size_t sia_workspace_size(int32_t op, const sia_seqmap* seq, int32_t K, int32_t heads,
                          int32_t latent_dim);

/* Empty batches: with seq->num_tokens == 0 every compute entry point returns
 * SIA_OK without launching anything once the scalar arguments (K, order,
 * method, dtypes and shapes) are valid; data pointers may then be NULL.       */

/* Static text for a sia_status value. */
const char* sia_status_string(int status);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char* sia_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SIA_H */

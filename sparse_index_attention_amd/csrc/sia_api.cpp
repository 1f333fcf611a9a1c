// libsia C ABI: host-side validation, workspace layout and dispatch.
// Every check happens before the first launch; kernels run asynchronously on
// the caller's stream and the library never synchronizes or allocates.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <string>

#include "sia_internal.hpp"

namespace sia {

static thread_local std::string g_last_hip_error;

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

int record_hip_error(hipError_t e) {
  g_last_hip_error = hipGetErrorString(e);
  return SIA_ERR_HIP;
}
static int hip_fail(hipError_t e) { return record_hip_error(e); }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A C caller may store any integer in a sia_dtype field; reading an
// out-of-range value through the C++ enum type is undefined, so the field is
// read as its raw integer and range-checked before any other use.
static bool dtype_known(const sia_dtype& d) {
  int32_t v;
  static_assert(sizeof(sia_dtype) == sizeof(int32_t), "sia_dtype is a 32-bit enum");
  std::memcpy(&v, &d, sizeof v);
  return v >= SIA_F32 && v <= SIA_MXFP8_E4M3;
}

static int check_seq(const sia_seqmap* s) {
  if (!s) return SIA_ERR_INVALID_ARG;
  if (s->num_tokens < 0) return SIA_ERR_INVALID_ARG;
  if (s->num_tokens == 0) return SIA_OK;
  if (!s->q_seq || !s->q_pos || !s->block_table) return SIA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->max_pages < 1 || s->num_pages < 1 || s->max_visible < 1) return SIA_ERR_INVALID_ARG;
  if (s->page_size != 64) return SIA_ERR_UNSUPPORTED;
  if ((int64_t)s->max_visible > (int64_t)s->max_pages * s->page_size) return SIA_ERR_INVALID_ARG;
  if ((int64_t)s->num_pages * s->page_size > INT32_MAX) return SIA_ERR_UNSUPPORTED;
  return SIA_OK;
}

// Shapes and dtypes always; pointers and their alignment only when there is
// work (num_tokens > 0).
static int check_indexer(const sia_indexer_in* in, int num_tokens = 1) {
  if (!in) return SIA_ERR_INVALID_ARG;
  if (!dtype_known(in->dtype)) return SIA_ERR_UNSUPPORTED;
  if (in->heads < 1 || in->dim < 1) return SIA_ERR_INVALID_ARG;
  const bool data = num_tokens > 0;
  if (data && (!in->q || !in->w || !in->k_pool)) return SIA_ERR_INVALID_ARG;
  if (in->q_bf16 != 0 && in->q_bf16 != 1) return SIA_ERR_INVALID_ARG;
  if (in->dtype == SIA_BF16) {
    if (in->q_bf16) return SIA_ERR_UNSUPPORTED;   // q already bfloat16
    if ((in->heads != 32 && in->heads != 64) || in->dim != 128) return SIA_ERR_UNSUPPORTED;
    if (data && (!aligned16(in->q) || !aligned16(in->k_pool))) return SIA_ERR_INVALID_ARG;
  } else if (in->dtype == SIA_F32) {
    if (in->q_bf16) return SIA_ERR_UNSUPPORTED;
    if (in->heads > 64 || (int64_t)in->heads * in->dim > 4096) return SIA_ERR_UNSUPPORTED;
  } else if (in->dtype == SIA_FP8_E4M3 || in->dtype == SIA_MXFP8_E4M3) {
    if (data && ((!in->q_bf16 && !in->q_scale) || !in->k_scale)) return SIA_ERR_INVALID_ARG;
    if ((in->heads != 32 && in->heads != 64) || in->dim != 128) return SIA_ERR_UNSUPPORTED;
    if (data && (!aligned16(in->q) || !aligned16(in->k_pool))) return SIA_ERR_INVALID_ARG;
    if (data && in->dtype == SIA_MXFP8_E4M3 &&
        ((!in->q_bf16 && (reinterpret_cast<uintptr_t>(in->q_scale) & 3u)) ||
         (reinterpret_cast<uintptr_t>(in->k_scale) & 3u)))
      return SIA_ERR_INVALID_ARG;
  } else {
    return SIA_ERR_UNSUPPORTED;
  }
  return SIA_OK;
}

static int check_scores(const float* scores, int64_t ld, const sia_seqmap* s) {
  if (s->num_tokens == 0) return SIA_OK;   // nothing is read
  if (!scores || !aligned16(scores)) return SIA_ERR_INVALID_ARG;
  if (ld < 1 || (ld & 3) != 0) return SIA_ERR_INVALID_ARG;
  if (s->num_tokens > 0 && ld < s->max_visible) return SIA_ERR_INVALID_ARG;
  return SIA_OK;
}

static int check_kv(const sia_kv_in* kv, sia_dtype q_dtype, int heads, int K) {
  if (!kv || !kv->kv_pool) return SIA_ERR_INVALID_ARG;
  if (!dtype_known(kv->dtype)) return SIA_ERR_UNSUPPORTED;
  if (K < 1) return SIA_ERR_INVALID_ARG;
  if (kv->latent_dim < 1 || kv->rope_dim < 0) return SIA_ERR_INVALID_ARG;
  if (kv->dtype == SIA_F32) {
    if (q_dtype != SIA_F32) return SIA_ERR_UNSUPPORTED;
    if (heads < 1 || heads > 64 || kv->latent_dim + kv->rope_dim > 1024 || K > kMaxTopK) return SIA_ERR_UNSUPPORTED;
    return SIA_OK;
  }
  if (kv->dtype != SIA_BF16 && kv->dtype != SIA_FP8_E4M3) return SIA_ERR_UNSUPPORTED;
  if (K > kMaxTopK) return SIA_ERR_UNSUPPORTED;
  if (q_dtype != SIA_BF16) return SIA_ERR_UNSUPPORTED;
  if (kv->latent_dim != 512 || kv->rope_dim != 64) return SIA_ERR_UNSUPPORTED;
  if (heads != 32 && heads != 64 && heads != 128) return SIA_ERR_UNSUPPORTED;
  if (!aligned16(kv->kv_pool)) return SIA_ERR_INVALID_ARG;
  if (kv->dtype == SIA_FP8_E4M3) {
    if (!kv->kv_scale) return SIA_ERR_INVALID_ARG;
    const bool page_tile = kv->scale_tokens == 64 && kv->scale_elems == 512;
    const bool tok_tile = kv->scale_tokens == 1 && kv->scale_elems == 128;
    if (!page_tile && !tok_tile) return SIA_ERR_UNSUPPORTED;
  }
  return SIA_OK;
}

static int mla_common(const void* q, sia_dtype q_dtype, int heads, const sia_kv_in* kv, const sia_seqmap* seq,
                      const int32_t* idx, int K, float scale, void* out) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_kv(kv, q_dtype, heads, K);
  if (rc) return rc;
  if (seq->num_tokens == 0) return SIA_OK;
  if (!q || !idx || !out) return SIA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return SIA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale != scale) return SIA_ERR_INVALID_ARG;
  return SIA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int64_t fused_ld(const sia_seqmap* s) { return ((int64_t)s->max_visible + 63) / 64 * 64; }

}  // namespace sia

using namespace sia;

// Method of sia_index_topk chosen by SIA_INDEX_TOPK_AUTO: on-chip ranges for
// decode-like batches (few queries per sequence) large enough to give every
// compute unit a (query, range) workgroup.
static int index_topk_auto(const sia_indexer_in& in, const sia_seqmap& seq) {
  if (in.dtype != SIA_FP8_E4M3 && in.dtype != SIA_MXFP8_E4M3) return SIA_INDEX_TOPK_SCORES;
  const int64_t wgs = (int64_t)seq.num_tokens * index_topk_ranges(seq.max_visible);
  return seq.num_tokens <= 2 * seq.batch && wgs >= num_cus() ? SIA_INDEX_TOPK_ONCHIP : SIA_INDEX_TOPK_SCORES;
}

// Workspace of either method: quantized queries (used when the caller passes
// bf16 queries; sized for the largest supported indexer, 64 heads x 128), then
// candidate lists (scores, positions) or the score matrix.
constexpr size_t kQCodesPerToken = 64 * 128, kQScalesPerToken = 64 * 4;
static size_t q_ws_bytes(const sia_seqmap& seq) {
  return align256((size_t)seq.num_tokens * kQCodesPerToken) + align256((size_t)seq.num_tokens * kQScalesPerToken);
}
// The score-matrix method keeps room for the block-aligned selection behind the matrix.
static size_t matrix_bytes(const sia_seqmap& seq) {
  return align256((size_t)seq.num_tokens * fused_ld(&seq) * sizeof(float));
}
static size_t index_topk_ws_bytes(const sia_seqmap& seq, int K) {
  const size_t cand = (size_t)seq.num_tokens * index_topk_ld(seq.max_visible, K);
  const size_t onchip = 2 * align256(cand * sizeof(float));
  const size_t matrix = matrix_bytes(seq) + topk_pages_ws_bytes(seq.num_tokens, seq.max_visible, K);
  return q_ws_bytes(seq) + (onchip > matrix ? onchip : matrix);
}

// Checks of K and `order` shared by the selecting entry points.
static int check_select(int K, int order) {
  if (K < 1 || order < SIA_ORDER_SCORE || order > SIA_SELECT_PAGES) return SIA_ERR_INVALID_ARG;
  if (order == SIA_SELECT_PAGES && K % 64 != 0) return SIA_ERR_INVALID_ARG;
  if (K > kMaxTopK) return SIA_ERR_UNSUPPORTED;
  return SIA_OK;
}

// With bf16 queries: quantize them into the workspace and describe the result
// in `out` (the caller's struct with q, q_scale pointing at the workspace).
static hipError_t prepare_q(const sia_indexer_in& in, const sia_seqmap& seq, void* ws, sia_indexer_in& out,
                            hipStream_t stream) {
  out = in;
  if (!in.q_bf16) return hipSuccess;
  unsigned char* codes = static_cast<unsigned char*>(ws);
  unsigned char* scales = codes + align256((size_t)seq.num_tokens * kQCodesPerToken);
  out.q = codes;
  out.q_scale = scales;
  out.q_scale_per_head = 0;
  out.q_bf16 = 0;
  return launch_quantize_q(in.q, seq.num_tokens, in.heads, in.dim, in.dtype == SIA_MXFP8_E4M3, codes, scales, stream);
}

static hipError_t run_index_topk(int method, const sia_indexer_in& in_given, const sia_seqmap& seq, int K,
                                 int order, int32_t* idx, float* vals, void* ws_all, hipStream_t stream) {
  sia_indexer_in in;
  hipError_t eq = prepare_q(in_given, seq, ws_all, in, stream);
  if (eq != hipSuccess) return eq;
  void* ws = static_cast<unsigned char*>(ws_all) + q_ws_bytes(seq);
  const SeqArgs s = seq_args(seq);
  if (method == SIA_INDEX_TOPK_ONCHIP) {
    const size_t cand = (size_t)seq.num_tokens * index_topk_ld(seq.max_visible, K);
    float* cscore = static_cast<float*>(ws);
    int32_t* cpos = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) + align256(cand * sizeof(float)));
    return launch_index_topk(in, s, K, order, idx, vals, cscore, cpos, stream);
  }
  float* scores = static_cast<float*>(ws);
  const int64_t ld = fused_ld(&seq);
  hipError_t e = launch_index_scores(in, s, scores, ld, stream);
  if (e != hipSuccess) return e;
  if (order == SIA_SELECT_PAGES)
    return launch_topk_pages(scores, ld, s, K, idx, vals, static_cast<unsigned char*>(ws) + matrix_bytes(seq), stream);
  return launch_topk(scores, ld, s, K, order, idx, vals, stream);
}

extern "C" {

const char* sia_status_string(int status) {
  switch (status) {
    case SIA_OK: return "ok";
    case SIA_ERR_INVALID_ARG: return "invalid argument";
    case SIA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SIA_ERR_WORKSPACE: return "workspace missing or too small";
    case SIA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* sia_last_hip_error(void) { return g_last_hip_error.c_str(); }

int sia_index_scores(const sia_indexer_in* in, const sia_seqmap* seq, float* scores, int64_t ld,
                     hipStream_t stream) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_indexer(in, seq->num_tokens);
  if (rc) return rc;
  rc = check_scores(scores, ld, seq);
  if (rc) return rc;
  if (in->q_bf16) return SIA_ERR_UNSUPPORTED;   // quantize first (sia_quantize_indexer_q)
  if (seq->num_tokens == 0) return SIA_OK;
  const hipError_t e = launch_index_scores(*in, seq_args(*seq), scores, ld, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

int sia_topk(const float* scores, int64_t ld, const sia_seqmap* seq, int32_t K, int32_t order, int32_t* idx,
             float* vals, hipStream_t stream) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_scores(scores, ld, seq);
  if (rc) return rc;
  if (K < 1 || K > kMaxTopK || (order != 0 && order != 1)) return K > kMaxTopK ? SIA_ERR_UNSUPPORTED : SIA_ERR_INVALID_ARG;
  if (seq->num_tokens == 0) return SIA_OK;
  if (!idx) return SIA_ERR_INVALID_ARG;
  const hipError_t e = launch_topk(scores, ld, seq_args(*seq), K, order, idx, vals, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

int sia_topk_pages(const float* scores, int64_t ld, const sia_seqmap* seq, int32_t K, int32_t* idx, float* vals,
                   void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_scores(scores, ld, seq);
  if (rc) return rc;
  rc = check_select(K, SIA_SELECT_PAGES);
  if (rc) return rc;
  if (seq->num_tokens == 0) return SIA_OK;
  if (!idx) return SIA_ERR_INVALID_ARG;
  const size_t need = sia_workspace_size(SIA_OP_TOPK_PAGES, seq, K, 1, 1);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SIA_ERR_WORKSPACE;
  const hipError_t e = launch_topk_pages(scores, ld, seq_args(*seq), K, idx, vals, ws, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

static int mla_entry(bool decode, const void* q, sia_dtype q_dtype, int32_t heads, const sia_kv_in* kv,
                     const sia_seqmap* seq, const int32_t* idx, int32_t K, float softmax_scale, void* out,
                     float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = mla_common(q, q_dtype, heads, kv, seq, idx, K, softmax_scale, out);
  if (rc) return rc;
  if (seq->num_tokens == 0) return SIA_OK;
  int splits = 1;
  if (decode && kv->dtype != SIA_F32) {
    splits = mla_splits(seq->num_tokens, K, heads);
    const size_t need = mla_workspace_bytes(seq->num_tokens, K, heads, kv->latent_dim);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return SIA_ERR_WORKSPACE;
  }
  const hipError_t e =
      launch_sparse_mla(q, heads, *kv, seq_args(*seq), idx, K, softmax_scale, out, lse, splits, ws, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

int sia_sparse_mla_decode(const void* q, sia_dtype q_dtype, int32_t heads, const sia_kv_in* kv,
                          const sia_seqmap* seq, const int32_t* idx, int32_t K, float softmax_scale, void* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return mla_entry(true, q, q_dtype, heads, kv, seq, idx, K, softmax_scale, out, lse, ws, ws_bytes, stream);
}

int sia_sparse_mla_prefill(const void* q, sia_dtype q_dtype, int32_t heads, const sia_kv_in* kv,
                           const sia_seqmap* seq, const int32_t* idx, int32_t K, float softmax_scale, void* out,
                           float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return mla_entry(false, q, q_dtype, heads, kv, seq, idx, K, softmax_scale, out, lse, ws, ws_bytes, stream);
}

size_t sia_workspace_size(int32_t op, const sia_seqmap* seq, int32_t K, int32_t heads, int32_t latent_dim) {
  if (check_seq(seq) != SIA_OK || K < 1 || heads < 1 || latent_dim < 1) return (size_t)-1;
  const int T = seq->num_tokens;
  switch (op) {
    case SIA_OP_TOPK:
    case SIA_OP_MLA_PREFILL:
      return 0;
    case SIA_OP_MLA_DECODE:
      return mla_workspace_bytes(T, K, heads, latent_dim);
    case SIA_OP_INDEX_TOPK:
      return T == 0 ? 0 : index_topk_ws_bytes(*seq, K);
    case SIA_OP_TOPK_PAGES:
      return T == 0 ? 0 : topk_pages_ws_bytes(T, seq->max_visible, K);
    case SIA_OP_INDEX_SELECT_ATTEND: {
      if (T == 0) return 0;
      const size_t scores = index_topk_ws_bytes(*seq, K);
      const size_t ids = align256((size_t)T * K * sizeof(int32_t));
      return scores + ids + align256(mla_workspace_bytes(T, K, heads, latent_dim));
    }
    default:
      return (size_t)-1;
  }
}

int sia_index_topk(const sia_indexer_in* in, const sia_seqmap* seq, int32_t K, int32_t order, int32_t method,
                   int32_t* idx, float* vals, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_indexer(in, seq->num_tokens);
  if (rc) return rc;
  if (method < SIA_INDEX_TOPK_AUTO || method > SIA_INDEX_TOPK_SCORES) return SIA_ERR_INVALID_ARG;
  rc = check_select(K, order);
  if (rc) return rc;
  if (method == SIA_INDEX_TOPK_ONCHIP &&
      ((in->dtype != SIA_FP8_E4M3 && in->dtype != SIA_MXFP8_E4M3) || order == SIA_SELECT_PAGES))
    return SIA_ERR_UNSUPPORTED;
  if (seq->num_tokens == 0) return SIA_OK;
  if (!idx) return SIA_ERR_INVALID_ARG;
  const size_t need = sia_workspace_size(SIA_OP_INDEX_TOPK, seq, K, 1, 1);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SIA_ERR_WORKSPACE;
  if (method == SIA_INDEX_TOPK_AUTO)
    method = order == SIA_SELECT_PAGES ? SIA_INDEX_TOPK_SCORES : index_topk_auto(*in, *seq);
  const hipError_t e = run_index_topk(method, *in, *seq, K, order, idx, vals, ws, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

int sia_quantize_indexer_q(const sia_indexer_in* in, int32_t num_tokens, void* q_codes, void* q_scales,
                           hipStream_t stream) {
  if (!in || !in->q || in->q_bf16 != 1 || num_tokens < 0 || !q_codes || !q_scales) return SIA_ERR_INVALID_ARG;
  if (!dtype_known(in->dtype)) return SIA_ERR_UNSUPPORTED;
  if (in->dtype != SIA_FP8_E4M3 && in->dtype != SIA_MXFP8_E4M3) return SIA_ERR_UNSUPPORTED;
  if ((in->heads != 32 && in->heads != 64) || in->dim != 128) return SIA_ERR_UNSUPPORTED;
  if (!aligned16(in->q) || !aligned16(q_codes) || (reinterpret_cast<uintptr_t>(q_scales) & 3u))
    return SIA_ERR_INVALID_ARG;
  if (num_tokens == 0) return SIA_OK;
  const hipError_t e = launch_quantize_q(in->q, num_tokens, in->heads, in->dim, in->dtype == SIA_MXFP8_E4M3,
                                         static_cast<uint8_t*>(q_codes), q_scales, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

int sia_index_topk_method(const sia_indexer_in* in, const sia_seqmap* seq) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_indexer(in, seq->num_tokens);
  if (rc) return rc;
  return index_topk_auto(*in, *seq);
}

int sia_index_select_attend(const sia_indexer_in* in, const void* q_mla, sia_dtype q_dtype, int32_t heads,
                            const sia_kv_in* kv, const sia_seqmap* seq, int32_t K, int32_t order,
                            float softmax_scale, int32_t* idx_out, void* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  int rc = check_seq(seq);
  if (rc) return rc;
  rc = check_indexer(in, seq->num_tokens);
  if (rc) return rc;
  rc = check_select(K, order);
  if (rc) return rc;
  rc = mla_common(q_mla, q_dtype, heads, kv, seq, idx_out ? idx_out : (const int32_t*)ws, K, softmax_scale, out);
  if (rc) return rc;
  if (seq->num_tokens == 0) return SIA_OK;
  const size_t need = sia_workspace_size(SIA_OP_INDEX_SELECT_ATTEND, seq, K, heads, kv->latent_dim);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SIA_ERR_WORKSPACE;
  const int T = seq->num_tokens;
  unsigned char* base = static_cast<unsigned char*>(ws);
  void* sel_ws = base;
  base += index_topk_ws_bytes(*seq, K);
  int32_t* ids = idx_out ? idx_out : reinterpret_cast<int32_t*>(base);
  base += align256((size_t)T * K * sizeof(int32_t));
  void* mla_ws = base;

  const SeqArgs s = seq_args(*seq);
  const int method = order == SIA_SELECT_PAGES ? SIA_INDEX_TOPK_SCORES : index_topk_auto(*in, *seq);
  hipError_t e = run_index_topk(method, *in, *seq, K, order, ids, nullptr, sel_ws, stream);
  if (e != hipSuccess) return hip_fail(e);
  const int splits = kv->dtype == SIA_F32 ? 1 : mla_splits(T, K, heads);
  e = launch_sparse_mla(q_mla, heads, *kv, s, ids, K, softmax_scale, out, lse, splits, mla_ws, stream);
  return e == hipSuccess ? SIA_OK : hip_fail(e);
}

}  // extern "C"

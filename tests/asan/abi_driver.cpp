// Drives every entry point of the C ABI layer through its validation and
// dispatch paths (host only; kernel launchers are stubs that count calls).
// Built with AddressSanitizer and UBSan by tests/test_abi_sanitizers.py.
// Every rejected call must return the documented status and launch nothing.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "sia.h"

extern int g_launches;
static int g_failures = 0;

#define EXPECT(call, want_rc, want_launch)                                                              \
  do {                                                                                                  \
    const int before = g_launches;                                                                      \
    const int rc = (call);                                                                              \
    const bool launched = g_launches > before;                                                          \
    if (rc != (want_rc) || launched != (want_launch)) {                                                 \
      std::printf("FAIL line %d: %s -> rc %d (want %d), launched %d (want %d)\n", __LINE__, #call, rc,  \
                  (int)(want_rc), (int)launched, (int)(want_launch));                                   \
      ++g_failures;                                                                                     \
    }                                                                                                   \
  } while (0)

// heap-allocated "device" buffers: never dereferenced by the stubs, but ASan
// sees any host-side overread of the argument structs
static void* buf(size_t n) { return std::aligned_alloc(256, (n + 255) / 256 * 256); }

static sia_seqmap* seqmap(int T, int max_visible = 4096) {
  auto* s = new sia_seqmap;
  s->q_seq = (const int32_t*)buf(4 * (T + 1));
  s->q_pos = (const int32_t*)buf(4 * (T + 1));
  s->block_table = (const int32_t*)buf(4 * 64);
  s->num_tokens = T;
  s->batch = 1;
  s->max_pages = 64;
  s->page_size = 64;
  s->num_pages = 64;
  s->max_visible = max_visible;
  return s;
}

static sia_indexer_in* indexer(sia_dtype dt = SIA_FP8_E4M3, int heads = 64) {
  auto* in = new sia_indexer_in;
  std::memset(in, 0, sizeof(*in));
  in->q = buf(1 << 20);
  in->q_scale = buf(1 << 16);
  in->w = (const float*)buf(1 << 16);
  in->k_pool = buf(1 << 20);
  in->k_scale = buf(1 << 16);
  in->dtype = dt;
  in->heads = heads;
  in->dim = dt == SIA_F32 ? 32 : 128;
  return in;
}

static sia_kv_in* kvin(sia_dtype dt = SIA_BF16) {
  auto* kv = new sia_kv_in;
  kv->kv_pool = buf(1 << 20);
  kv->kv_scale = dt == SIA_FP8_E4M3 ? (const float*)buf(1 << 12) : nullptr;
  kv->dtype = dt;
  kv->scale_tokens = 64;
  kv->scale_elems = 512;
  kv->latent_dim = 512;
  kv->rope_dim = 64;
  return kv;
}

int main() {
  const int T = 8, K = 256;
  sia_seqmap* seq = seqmap(T);
  sia_seqmap* empty = seqmap(0);
  sia_indexer_in* ix = indexer();
  float* scores = (float*)buf((size_t)T * 4096 * 4);
  int32_t* idx = (int32_t*)buf((size_t)T * K * 4);
  float* vals = (float*)buf((size_t)T * K * 4);

  // status strings
  for (int c = -5; c <= 1; ++c)
    if (!sia_status_string(c)) ++g_failures;

  // ---- sia_index_scores
  EXPECT(sia_index_scores(nullptr, seq, scores, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_index_scores(ix, nullptr, scores, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_index_scores(ix, seq, scores, 4096, nullptr), SIA_OK, true);
  EXPECT(sia_index_scores(ix, seq, scores, 4095, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_index_scores(ix, seq, scores, 2048, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_index_scores(ix, seq, scores + 1, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_index_scores(ix, empty, nullptr, 4096, nullptr), SIA_OK, false);
  {
    sia_seqmap s2 = *seq;
    s2.page_size = 32;
    EXPECT(sia_index_scores(ix, &s2, scores, 4096, nullptr), SIA_ERR_UNSUPPORTED, false);
    s2 = *seq;
    s2.max_visible = 64 * 64 + 1;
    EXPECT(sia_index_scores(ix, &s2, scores, 8192, nullptr), SIA_ERR_INVALID_ARG, false);
    s2 = *seq;
    s2.num_tokens = -1;
    EXPECT(sia_index_scores(ix, &s2, scores, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
    s2 = *seq;
    s2.q_pos = nullptr;
    EXPECT(sia_index_scores(ix, &s2, scores, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
  }
  {
    sia_indexer_in i2 = *ix;
    i2.heads = 48;
    EXPECT(sia_index_scores(&i2, seq, scores, 4096, nullptr), SIA_ERR_UNSUPPORTED, false);
    i2 = *ix;
    i2.q_bf16 = 1;
    EXPECT(sia_index_scores(&i2, seq, scores, 4096, nullptr), SIA_ERR_UNSUPPORTED, false);
    i2 = *ix;
    i2.k_scale = nullptr;
    EXPECT(sia_index_scores(&i2, seq, scores, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
    i2 = *ix;
    i2.dtype = (sia_dtype)9;
    EXPECT(sia_index_scores(&i2, seq, scores, 4096, nullptr), SIA_ERR_UNSUPPORTED, false);
    i2 = *ix;
    i2.dtype = SIA_MXFP8_E4M3;
    i2.k_scale = (const char*)ix->k_scale + 1;
    EXPECT(sia_index_scores(&i2, seq, scores, 4096, nullptr), SIA_ERR_INVALID_ARG, false);
  }

  // ---- sia_topk
  EXPECT(sia_topk(scores, 4096, seq, K, 0, idx, vals, nullptr), SIA_OK, true);
  EXPECT(sia_topk(scores, 4096, seq, K, 1, idx, nullptr, nullptr), SIA_OK, true);
  EXPECT(sia_topk(scores, 4096, seq, 0, 0, idx, vals, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_topk(scores, 4096, seq, 4096, 0, idx, vals, nullptr), SIA_ERR_UNSUPPORTED, false);
  EXPECT(sia_topk(scores, 4096, seq, K, 2, idx, vals, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_topk(scores, 4096, seq, K, 0, nullptr, vals, nullptr), SIA_ERR_INVALID_ARG, false);
  EXPECT(sia_topk(nullptr, 4096, empty, K, 0, nullptr, nullptr, nullptr), SIA_OK, false);

  // ---- sia_topk_pages
  {
    const size_t need = sia_workspace_size(SIA_OP_TOPK_PAGES, seq, K, 1, 1);
    void* ws = buf(need);
    EXPECT(sia_topk_pages(scores, 4096, seq, K, idx, vals, ws, need, nullptr), SIA_OK, true);
    EXPECT(sia_topk_pages(scores, 4096, seq, K, idx, vals, ws, need - 1, nullptr), SIA_ERR_WORKSPACE, false);
    EXPECT(sia_topk_pages(scores, 4096, seq, K, idx, vals, (char*)ws + 16, need, nullptr), SIA_ERR_WORKSPACE, false);
    EXPECT(sia_topk_pages(scores, 4096, seq, 100, idx, vals, ws, need, nullptr), SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_topk_pages(scores, 4096, seq, K, nullptr, vals, ws, need, nullptr), SIA_ERR_INVALID_ARG, false);
    std::free(ws);
  }

  // ---- sia_index_topk (+ method query)
  {
    const size_t need = sia_workspace_size(SIA_OP_INDEX_TOPK, seq, K, 1, 1);
    void* ws = buf(need);
    for (int method = 0; method <= 2; ++method)
      EXPECT(sia_index_topk(ix, seq, K, 0, method, idx, vals, ws, need, nullptr), SIA_OK, true);
    EXPECT(sia_index_topk(ix, seq, K, 0, 3, idx, vals, ws, need, nullptr), SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_index_topk(ix, seq, K, SIA_SELECT_PAGES, SIA_INDEX_TOPK_ONCHIP, idx, vals, ws, need, nullptr),
           SIA_ERR_UNSUPPORTED, false);
    EXPECT(sia_index_topk(ix, seq, K, 0, 0, idx, vals, ws, need - 1, nullptr), SIA_ERR_WORKSPACE, false);
    EXPECT(sia_index_topk(ix, seq, K, 0, 0, idx, vals, nullptr, 0, nullptr), SIA_ERR_WORKSPACE, false);
    sia_indexer_in f32 = *indexer(SIA_F32, 4);
    EXPECT(sia_index_topk(&f32, seq, K, 0, SIA_INDEX_TOPK_ONCHIP, idx, vals, ws, need, nullptr), SIA_ERR_UNSUPPORTED,
           false);
    sia_indexer_in qb = *ix;
    qb.q_bf16 = 1;
    qb.q_scale = nullptr;
    EXPECT(sia_index_topk(&qb, seq, K, 0, 0, idx, vals, ws, need, nullptr), SIA_OK, true);
    const int m = sia_index_topk_method(ix, seq);
    if (m != SIA_INDEX_TOPK_ONCHIP && m != SIA_INDEX_TOPK_SCORES) ++g_failures;
    if (sia_index_topk_method(nullptr, seq) >= 0) ++g_failures;
    std::free(ws);
  }

  // ---- sia_quantize_indexer_q
  {
    sia_indexer_in qb = *ix;
    qb.q_bf16 = 1;
    void* codes = buf((size_t)T * 64 * 128);
    void* qs = buf((size_t)T * 64 * 4 * 4);
    EXPECT(sia_quantize_indexer_q(&qb, T, codes, qs, nullptr), SIA_OK, true);
    EXPECT(sia_quantize_indexer_q(ix, T, codes, qs, nullptr), SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_quantize_indexer_q(&qb, -1, codes, qs, nullptr), SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_quantize_indexer_q(&qb, 0, codes, qs, nullptr), SIA_OK, false);
    EXPECT(sia_quantize_indexer_q(&qb, T, (char*)codes + 8, qs, nullptr), SIA_ERR_INVALID_ARG, false);
    qb.heads = 16;
    EXPECT(sia_quantize_indexer_q(&qb, T, codes, qs, nullptr), SIA_ERR_UNSUPPORTED, false);
  }

  // ---- sparse MLA, both entry points
  {
    sia_kv_in* kv = kvin();
    void* q = buf((size_t)T * 128 * 576 * 2);
    void* out = buf((size_t)T * 128 * 512 * 2);
    float* lse = (float*)buf((size_t)T * 128 * 4);
    const float sc = 1.f / 24.f;
    const size_t need = sia_workspace_size(SIA_OP_MLA_DECODE, seq, K, 128, 512);
    void* ws = need ? buf(need) : nullptr;
    EXPECT(sia_sparse_mla_decode(q, SIA_BF16, 128, kv, seq, idx, K, sc, out, lse, ws, need, nullptr), SIA_OK, true);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, kv, seq, idx, K, sc, out, nullptr, nullptr, 0, nullptr), SIA_OK,
           true);
    if (need)
      EXPECT(sia_sparse_mla_decode(q, SIA_BF16, 128, kv, seq, idx, K, sc, out, lse, ws, need - 1, nullptr),
             SIA_ERR_WORKSPACE, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 96, kv, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_UNSUPPORTED, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, kv, seq, idx, K, NAN, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, kv, seq, idx, K, 0.f, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, kv, seq, idx, 0, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, kv, seq, idx, 4096, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_UNSUPPORTED, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, nullptr, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, kv, seq, nullptr, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_sparse_mla_prefill(q, SIA_F32, 128, kv, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_UNSUPPORTED, false);
    EXPECT(sia_sparse_mla_prefill((char*)q + 2, SIA_BF16, 128, kv, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_sparse_mla_prefill(nullptr, SIA_BF16, 128, kv, empty, nullptr, K, sc, nullptr, nullptr, nullptr, 0,
                                  nullptr),
           SIA_OK, false);
    sia_kv_in k2 = *kv;
    k2.latent_dim = 256;
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, &k2, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_UNSUPPORTED, false);
    sia_kv_in* f8 = kvin(SIA_FP8_E4M3);
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, f8, seq, idx, K, sc, out, lse, nullptr, 0, nullptr), SIA_OK, true);
    f8->scale_tokens = 1;
    f8->scale_elems = 128;
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, f8, seq, idx, K, sc, out, lse, nullptr, 0, nullptr), SIA_OK, true);
    f8->scale_tokens = 32;
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, f8, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_UNSUPPORTED, false);
    f8->scale_tokens = 64;
    f8->scale_elems = 512;
    f8->kv_scale = nullptr;
    EXPECT(sia_sparse_mla_prefill(q, SIA_BF16, 128, f8, seq, idx, K, sc, out, lse, nullptr, 0, nullptr),
           SIA_ERR_INVALID_ARG, false);

    // ---- the whole path in one call
    const size_t need_all = sia_workspace_size(SIA_OP_INDEX_SELECT_ATTEND, seq, K, 128, 512);
    void* wsa = buf(need_all);
    EXPECT(sia_index_select_attend(ix, q, SIA_BF16, 128, kv, seq, K, 0, sc, idx, out, lse, wsa, need_all, nullptr),
           SIA_OK, true);
    EXPECT(sia_index_select_attend(ix, q, SIA_BF16, 128, kv, seq, K, 0, sc, nullptr, out, lse, wsa, need_all, nullptr),
           SIA_OK, true);
    EXPECT(sia_index_select_attend(ix, q, SIA_BF16, 128, kv, seq, K, SIA_SELECT_PAGES, sc, idx, out, lse, wsa,
                                   need_all, nullptr),
           SIA_OK, true);
    EXPECT(sia_index_select_attend(ix, q, SIA_BF16, 128, kv, seq, K, 0, sc, idx, out, lse, wsa, need_all - 1, nullptr),
           SIA_ERR_WORKSPACE, false);
    EXPECT(sia_index_select_attend(ix, q, SIA_BF16, 128, kv, seq, K, 3, sc, idx, out, lse, wsa, need_all, nullptr),
           SIA_ERR_INVALID_ARG, false);
    EXPECT(sia_index_select_attend(ix, nullptr, SIA_BF16, 128, kv, empty, K, 0, sc, nullptr, nullptr, nullptr, nullptr,
                                   0, nullptr),
           SIA_OK, false);
    std::free(wsa);
  }

  // ---- workspace sizes: invalid arguments and the largest shapes the ABI admits
  if (sia_workspace_size(99, seq, K, 128, 512) != (size_t)-1) ++g_failures;
  if (sia_workspace_size(SIA_OP_TOPK, nullptr, K, 128, 512) != (size_t)-1) ++g_failures;
  if (sia_workspace_size(SIA_OP_MLA_DECODE, seq, 0, 128, 512) != (size_t)-1) ++g_failures;
  {
    sia_seqmap big = *seq;
    big.num_tokens = 1 << 20;
    big.max_pages = (1 << 25) / 64;
    big.num_pages = (1 << 25) / 64;
    big.max_visible = 1 << 25;
    for (int op = 0; op <= 5; ++op) {
      const size_t n = sia_workspace_size(op, &big, 2048, 128, 512);
      if (n == (size_t)-1) ++g_failures;
    }
  }
  std::printf("%s: %d failures\n", g_failures ? "abi driver FAILED" : "abi driver ok", g_failures);
  return g_failures ? 1 : 0;
}

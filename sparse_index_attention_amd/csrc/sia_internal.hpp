// Host-side declarations shared between the C ABI layer and the kernel sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sia.h"

namespace sia {

// Plain copy of the sequence map handed to every kernel.
struct SeqArgs {
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* block_table;
  int32_t T;
  int32_t batch;
  int32_t max_pages;
  int32_t num_pages;
  int32_t max_visible;
};

inline SeqArgs seq_args(const sia_seqmap& s) {
  return SeqArgs{s.q_seq, s.q_pos, s.block_table, s.num_tokens, s.batch, s.max_pages, s.num_pages, s.max_visible};
}

int num_cus();
// Records e as the text sia_last_hip_error returns; gives SIA_ERR_HIP.
int record_hip_error(hipError_t e);

// indexer.hip
hipError_t launch_index_scores(const sia_indexer_in& in, const SeqArgs& s, float* scores, int64_t ld,
                               hipStream_t st);
// topk.hip
// Candidate lists of the fused score + Top-K pass: row t holds, in ascending
// position order, the best min(K, keys) entries of each range of range_keys
// keys; pos[t * ld + i] is the position of entry i.  pos == nullptr: plain rows.
struct CandMap {
  const int32_t* pos;
  int range_keys;
  int K;
};
hipError_t launch_topk(const float* scores, int64_t ld, const SeqArgs& s, int K, int order, int32_t* idx,
                       float* vals, hipStream_t st);
hipError_t launch_topk_candidates(const float* cscore, const int32_t* cpos, int64_t ldc, int range_keys,
                                  const SeqArgs& s, int K, int order, int32_t* idx, float* vals, hipStream_t st);
// topk_pages.hip: block-aligned selection (whole 64-position pages, ascending)
int64_t topk_pages_ld(int max_visible);
size_t topk_pages_ws_bytes(int T, int max_visible, int K);
hipError_t launch_topk_pages(const float* scores, int64_t ld, const SeqArgs& s, int K, int32_t* idx, float* vals,
                             void* ws, hipStream_t st);
// indexer_bf16.hip
hipError_t launch_index_scores_bf16(const sia_indexer_in& in, const SeqArgs& s, float* scores, int64_t ld,
                                    hipStream_t st);
// quantize.hip
hipError_t launch_quantize_q(const void* q_bf16, int T, int heads, int dim, bool mx, uint8_t* codes, void* scales,
                             hipStream_t st);
// index_topk.hip
constexpr int kIndexTopkRangeKeys = 8192;
constexpr int kMaxTopK = 2048;  // largest K any entry point accepts
int index_topk_ranges(int max_visible);
// leading dimension of the candidate lists (a multiple of 4 floats)
int64_t index_topk_ld(int max_visible, int K);
hipError_t launch_index_topk(const sia_indexer_in& in, const SeqArgs& s, int K, int order, int32_t* idx,
                             float* vals, float* cscore, int32_t* cpos, hipStream_t st);
// sparse_mla.hip
int mla_splits(int T, int K, int heads);
size_t mla_workspace_bytes(int T, int K, int heads, int latent);
hipError_t launch_sparse_mla(const void* q, int heads, const sia_kv_in& kv, const SeqArgs& s,
                             const int32_t* idx, int K, float scale, void* out, float* lse, int splits,
                             void* ws, hipStream_t st);

}  // namespace sia

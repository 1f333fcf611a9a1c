// Step 1 — indexer scores.
//
//   scores[t, s] = sum_h w[t,h] * ReLU(qs[t,h] * ks[s] * <q[t,h], k[s]>),  s <= q_pos[t]
//
// [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models",
//      section "Sparse Attention Pipeline Optimization": the indexer scores each
//      history position from the paged key cache and weights the heads.
// [P2] "Efficient Inference Deployment and Optimization for Hybrid Attention
//      LLMs", section 3.1: scoring, head weighting and Top-K form the index stage.
// [P3] "Day-One Inference Adaptation for Very Large Hybrid-Attention Models",
//      section 3.1: the causal mask is generated inside the scoring kernel.
//
// fp8 path (gfx950): q.k over all keys is a dense contraction, so it runs on
// v_mfma_f32_32x32x64_f8f6f4 (OCP e4m3 inputs, fp32 accumulate).  Per wave:
// the query's indexer heads sit in the MFMA M dimension (held in registers for
// the whole key range), 32 keys per N tile, depth 128 = two K steps.  The
// epilogue applies ReLU and the per-head weight (with the query scale folded
// in) in registers, reduces across heads with one cross-lane exchange, scales
// by the key's scale and writes one coalesced row segment per 64-key page.
// Since scales are positive, ReLU(qs*ks*d) = qs*ks*ReLU(d), which is what makes
// this folding exact in real arithmetic.
#include "index_core.hpp"

namespace sia {

// ---------------------------------------------------------------------------
// float32 path: small head counts / dims, one thread per key.
// ---------------------------------------------------------------------------
constexpr int kF32MaxQ = 4096;  // heads * dim

__global__ __launch_bounds__(256) void k_index_scores_f32(IndexArgs a) {
  __shared__ float sq[kF32MaxQ];
  __shared__ float sw[64];
  const int t = blockIdx.x;
  const int H = a.H, D = a.D;
  const int pos = clampi(a.s.q_pos[t], -1, a.s.max_visible - 1);
  const int b = clampi(a.s.q_seq[t], 0, a.s.batch - 1);
  const float* q = (const float*)a.q + (int64_t)t * H * D;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) sq[i] = q[i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) sw[i] = a.w[(int64_t)t * H + i];
  __syncthreads();
  const int s = blockIdx.y * blockDim.x + threadIdx.x;
  if (s >= a.s.max_visible) return;
  float out = -INFINITY;
  if (s <= pos) {
    const int64_t slot = page_slot(a.s.block_table + (int64_t)b * a.s.max_pages, s, a.s.num_pages);
    const float* k = (const float*)a.k_pool + slot * D;
    out = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[h * D + d], k[d], dot);
      out = fmaf(sw[h], fmaxf(dot, 0.f), out);
    }
  }
  a.scores[(int64_t)t * a.ld + s] = out;
}

// ---------------------------------------------------------------------------
// fp8 path: MFMA 32x32x64, dim 128, HI in {32, 64}.
// ---------------------------------------------------------------------------
// One wave = one query row x a range of 64-key pages.
// Lane l: nn = l % 32 (key within an N tile / head within an M tile), hh = l / 32.
// K-step mapping (same for both operands): step st of lane half hh covers
// depth bytes [64*hh + 32*st, 64*hh + 32*st + 32).
template <int HI>
__global__ __launch_bounds__(256, 2) void k_index_scores_fp8(IndexArgs a, int n_qblocks, int n_chunks,
                                                             int chunks_per_item) {
  const int wave = threadIdx.x >> 6;
  const int n_ranges = (n_chunks + chunks_per_item - 1) / chunks_per_item;
  const int64_t items = (int64_t)n_qblocks * n_ranges;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    // heaviest (latest) query blocks first
    const int qb = n_qblocks - 1 - (int)(it / n_ranges);
    const int rg = (int)(it % n_ranges);
    const int t = qb * 4 + wave;
    if (t >= a.s.T) continue;
    const int pos = clampi(a.s.q_pos[t], -1, a.s.max_visible - 1);
    const int b = clampi(a.s.q_seq[t], 0, a.s.batch - 1);
    const int c_begin = rg * chunks_per_item;
    int c_end = c_begin + chunks_per_item;
    c_end = c_end < n_chunks ? c_end : n_chunks;
    const int c_vis = (pos >> 6) + 1;  // pages holding a visible key
    c_end = c_end < c_vis ? c_end : c_vis;
    if (c_begin >= c_end) continue;

    float* srow = a.scores + (int64_t)t * a.ld;
    score_pages<HI>(a, t, pos, b, c_begin, c_end, [&](int s, float score) __attribute__((always_inline)) {
      if (s < a.s.max_visible) srow[s] = score;
    });
  }
}

hipError_t launch_index_scores(const sia_indexer_in& in, const SeqArgs& s, float* scores, int64_t ld,
                               hipStream_t st) {
  IndexArgs a{in.q, in.q_scale, in.w, in.k_pool, in.k_scale, in.q_scale_per_head, in.heads, in.dim, s, scores, ld};
  if (s.T == 0 || s.max_visible == 0) return hipSuccess;
  if (in.dtype == SIA_F32) {
    dim3 grid(s.T, (s.max_visible + 255) / 256);
    hipLaunchKernelGGL(k_index_scores_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int n_qblocks = (s.T + 3) / 4;
  const int n_chunks = (s.max_visible + 63) / 64;
  // enough waves to keep every CU busy: split the key range of each query
  // block when there are few query blocks (decode), keep it whole otherwise
  const int cus = num_cus();
  const int64_t target_items = (int64_t)cus * 2;
  int n_ranges = (int)((target_items + n_qblocks - 1) / n_qblocks);
  n_ranges = n_ranges < 1 ? 1 : (n_ranges > n_chunks ? n_chunks : n_ranges);
  const int cpi = (n_chunks + n_ranges - 1) / n_ranges;
  const int64_t items = (int64_t)n_qblocks * ((n_chunks + cpi - 1) / cpi);
  const int64_t resident = (int64_t)cus * 2;
  const int grid = (int)(items < resident ? items : resident);
  if (in.heads == 64)
    hipLaunchKernelGGL(k_index_scores_fp8<64>, dim3(grid), dim3(256), 0, st, a, n_qblocks, n_chunks, cpi);
  else
    hipLaunchKernelGGL(k_index_scores_fp8<32>, dim3(grid), dim3(256), 0, st, a, n_qblocks, n_chunks, cpi);
  return hipGetLastError();
}

}  // namespace sia

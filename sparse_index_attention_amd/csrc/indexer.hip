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
#include "sia_common.hpp"
#include "sia_internal.hpp"

namespace sia {

struct IndexArgs {
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k_pool;
  const float* k_scale;
  int q_scale_per_head;
  int H;
  int D;
  SeqArgs s;
  float* scores;
  int64_t ld;
};

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
__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One wave = one query row x a range of 64-key pages.
// Lane l: nn = l % 32 (key within an N tile / head within an M tile), hh = l / 32.
// K-step mapping (same for both operands): step st of lane half hh covers
// depth bytes [64*hh + 32*st, 64*hh + 32*st + 32).
template <int HI>
__global__ __launch_bounds__(256, 2) void k_index_scores_fp8(IndexArgs a, int n_qblocks, int n_chunks,
                                                             int chunks_per_item) {
  constexpr int MT = HI / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, nn = lane & 31;
  const int n_ranges = (n_chunks + chunks_per_item - 1) / chunks_per_item;
  const int64_t items = (int64_t)n_qblocks * n_ranges;
  const uint8_t* __restrict__ kpool = (const uint8_t*)a.k_pool;
  const uint8_t* __restrict__ qbase = (const uint8_t*)a.q;

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

    const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;
    float* srow = a.scores + (int64_t)t * a.ld;

    // key pages go through a ring of three register buffers: while page c is
    // computed, pages c+1 and c+2 are in flight
    auto load_page = [&](int c, v8i (&kb)[2][2], float& ks) __attribute__((always_inline)) {
      int page = table[c];
      page = page < 0 ? 0 : (page >= a.s.num_pages ? a.s.num_pages - 1 : page);
      const uint8_t* pb = kpool + (int64_t)page * (kPage * 128) + 64 * hh;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint8_t* kr = pb + (32 * kt + nn) * 128;
        kb[kt][0] = *(const v8i*)(kr);
        kb[kt][1] = *(const v8i*)(kr + 32);
      }
      ks = a.k_scale[(int64_t)page * kPage + lane];
    };
    v8i k0[2][2], k1[2][2], k2[2][2];
    float ks0 = 0.f, ks1 = 0.f, ks2 = 0.f;
    load_page(c_begin, k0, ks0);
    if (c_begin + 1 < c_end) load_page(c_begin + 1, k1, ks1);
    if (c_begin + 2 < c_end) load_page(c_begin + 2, k2, ks2);

    // query operand (A): head m = 32*mt + nn
    v8i qa[MT][2];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* qr = qbase + ((int64_t)t * HI + 32 * mt + nn) * 128 + 64 * hh;
      qa[mt][0] = *(const v8i*)(qr);
      qa[mt][1] = *(const v8i*)(qr + 32);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int head = 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float qs = a.q_scale_per_head ? a.q_scale[(int64_t)t * HI + head] : a.q_scale[t];
        wr[mt][r] = a.w[(int64_t)t * HI + head] * qs;
      }
    }
    // scores of page c from buffer kb, then buffer kb takes page c+3
    auto step = [&](int c, v8i (&kb)[2][2], float& ks) __attribute__((always_inline)) {
      float p[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float sum = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          v16f acc = {};
          acc = mfma_f8(qa[mt][0], kb[kt][0], acc);
          acc = mfma_f8(qa[mt][1], kb[kt][1], acc);
#pragma unroll
          for (int r = 0; r < 16; ++r) sum = fmaf(wr[mt][r], fmaxf(acc[r], 0.f), sum);
        }
        p[kt] = sum;
      }
      // lane half hh keeps key tile hh; lane l ends with key 64*c + l
      const float mine = hh ? p[1] : p[0];
      const float give = hh ? p[0] : p[1];
      float score = (mine + __shfl_xor(give, 32, 64)) * ks;
      const int s = c * 64 + lane;
      if (s > pos) score = -INFINITY;
      if (s < a.s.max_visible) srow[s] = score;
      if (c + 3 < c_end) load_page(c + 3, kb, ks);
    };
    int c = c_begin;
    for (; c + 3 <= c_end; c += 3) {
      step(c, k0, ks0);
      step(c + 1, k1, ks1);
      step(c + 2, k2, ks2);
    }
    if (c < c_end) step(c, k0, ks0);
    if (c + 1 < c_end) step(c + 1, k1, ks1);
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

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
#include "block_prims.hpp"
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
template <int HI, bool MX>
__global__ __launch_bounds__(256, 2) void k_index_scores_fp8(IndexArgs a, int n_qblocks, int n_chunks,
                                                             int chunks_per_item) {
  // wave-uniform values are kept in scalar registers (readfirstlane), so that
  // the page and row descriptors built from them are scalar too
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n_ranges = (n_chunks + chunks_per_item - 1) / chunks_per_item;
  const int64_t items = (int64_t)n_qblocks * n_ranges;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    // heaviest (latest) query blocks first
    const int qb = n_qblocks - 1 - (int)(it / n_ranges);
    const int rg = (int)(it % n_ranges);
    const int t = qb * 4 + wave;
    if (t >= a.s.T) continue;
    const int pos = __builtin_amdgcn_readfirstlane(clampi(a.s.q_pos[t], -1, a.s.max_visible - 1));
    const int b = __builtin_amdgcn_readfirstlane(clampi(a.s.q_seq[t], 0, a.s.batch - 1));
    const int c_begin = rg * chunks_per_item;
    int c_end = c_begin + chunks_per_item;
    c_end = c_end < n_chunks ? c_end : n_chunks;
    const int c_vis = (pos >> 6) + 1;  // pages holding a visible key
    c_end = c_end < c_vis ? c_end : c_vis;
    if (c_begin >= c_end) continue;

    float* srow = a.scores + (int64_t)t * a.ld;
    score_pages<HI, MX>(a, t, pos, b, c_begin, c_end, [&](int s, float score) __attribute__((always_inline)) {
      // a descriptor over the row from this page on, ending at max_visible:
      // its range check drops the stores past the row's end, with no branch
      const int s0 = __builtin_amdgcn_readfirstlane(s) & ~63;   // 64c (lane 0 holds key 64c)
      const uint64_t ra = (uint64_t)(uintptr_t)(srow + s0);
      void* rp = (void*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ra >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ra));
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(rp, 0, (a.s.max_visible - s0) * 4, kRawBuffer);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), prs, (s - s0) * 4, 0, 0);
    });
  }
}

// ---------------------------------------------------------------------------
// fp8 path, several queries per sequence (prefill): the kSQ queries of a
// workgroup share each key page through LDS instead of each wave reading it
// from the cache hierarchy on its own.  One workgroup = kSQ consecutive
// queries x a chunk of kSChunk pages; chunks run in order across the grid, so
// the chunk in flight stays in every L2.  A workgroup whose queries belong to
// different sequences lets each wave score its own query's pages.
// ---------------------------------------------------------------------------
constexpr int kSQ = 4;
constexpr int kSChunk = 128;
constexpr int kSThreads = 64 * kSQ;

// Byte offset of 16-byte chunk j (0..7) of key row r in an LDS page: chunk j
// is stored at j ^ ((r >> 1) & 7), so the 16 lanes of one read phase (rows
// r..r+15 at the same j) fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kswz(int r, int j) { return r * 128 + 16 * (j ^ ((r >> 1) & 7)); }

struct KStage {  // one thread's share of a key page in flight: 32 bytes and a scale
  uint4 x, y;
  float s;
};

template <int HI, bool MX>
__global__ __launch_bounds__(kSThreads, 3) void k_index_scores_fp8_shared(IndexArgs a, int n_qblocks) {
  constexpr int MT = HI / 32;
  __shared__ __attribute__((aligned(16))) uint8_t kl[2][kPage * 128];
  __shared__ float kls[2][kPage];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, nn = lane & 31;
  const int ch = (int)blockIdx.x / n_qblocks;
  const int t0 = (n_qblocks - 1 - (int)blockIdx.x % n_qblocks) * kSQ;

  // The block's queries (the same values in every thread).  Queries of one
  // sequence share its pages; a block that spans sequences takes one round per
  // sequence, in which only that sequence's waves compute.
  const int nq = min(kSQ, a.s.T - t0);
  int qseq[kSQ], cvis[kSQ], cmax = 0;
#pragma unroll
  for (int i = 0; i < kSQ; ++i) {
    qseq[i] = i < nq ? clampi(a.s.q_seq[t0 + i], 0, a.s.batch - 1) : -1;
    cvis[i] = i < nq ? (clampi(a.s.q_pos[t0 + i], -1, a.s.max_visible - 1) >> 6) + 1 : 0;
    cmax = max(cmax, cvis[i]);
  }
  const int c_begin = ch * kSChunk;
  if (c_begin >= cmax) return;

  const int t = t0 + wave;
  const bool has_q = wave < nq;
  const int pos = has_q ? clampi(a.s.q_pos[t], -1, a.s.max_visible - 1) : -1;
  const int my_seq = has_q ? clampi(a.s.q_seq[t], 0, a.s.batch - 1) : -1;
  const int c_own = (pos >> 6) + 1;
  float* const srow = a.scores + (int64_t)(has_q ? t : 0) * a.ld;
  const uint8_t* __restrict__ kpool = (const uint8_t*)a.k_pool;
  const int sr = tid >> 2, sj = 2 * (tid & 3);  // thread moves row sr, chunks sj and sj+1
  // Per-lane parts of every address are fixed for the whole kernel; the
  // per-page parts are wave-uniform and go into buffer descriptors built with
  // scalar arithmetic, so the page loop spends its vector instructions on the
  // scores themselves.
  const int kvoff = sr * 128 + 16 * sj;    // this thread's bytes of a key page
  // LDS read bases of the key operand: key row 32kt + nn (kt adds 4096 bytes),
  // 16-byte chunk j at j ^ ((row >> 1) & 7), the same swizzle for both kt
  int kbase[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      // 16-byte chunks of the row this lane feeds (see mx_operand for MX)
      const int j = MX ? 4 * st + 2 * x + hh : 4 * hh + 2 * st + x;
      kbase[st][x] = kswz(nn, j);
    }

  // ---- this wave's query (operand A) and folded head weights
  v8i qa[MT][2];
  uint32_t qsc[MT];   // MX: group scales of head 32mt + nn
  float wr[MT][16];
  if (has_q) {
    const uint8_t* __restrict__ qbase = (const uint8_t*)a.q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* qr = qbase + ((int64_t)t * HI + 32 * mt + nn) * 128;
      if constexpr (MX) {
        qa[mt][0] = mx_operand<0>(qr, hh);
        qa[mt][1] = mx_operand<1>(qr, hh);
        qsc[mt] = mx_lane_scales(*(const uint32_t*)(a.q_mx + ((int64_t)t * HI + 32 * mt + nn) * 4), hh);
      } else {
        qa[mt][0] = *(const v8i*)(qr + 64 * hh);
        qa[mt][1] = *(const v8i*)(qr + 64 * hh + 32);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int head = 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        float qs = 1.f;
        if constexpr (!MX) qs = a.q_scale_per_head ? a.q_scale[(int64_t)t * HI + head] : a.q_scale[t];
        wr[mt][r] = a.w[(int64_t)t * HI + head] * qs;
      }
    }
  }

  // scores of page c from LDS buffer `cur` (same arithmetic as score_pages)
  auto compute = [&](int c, int cur) __attribute__((always_inline)) {
    v8i kb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint4 lo = *(const uint4*)&kl[cur][kbase[st][0] + 4096 * kt];
        const uint4 hi = *(const uint4*)&kl[cur][kbase[st][1] + 4096 * kt];
        kb[kt][st] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
    // fp8: key scale of key `lane`; MX: the staged words hold each key's four
    // group-scale bytes
    const float ks = kls[cur][lane];
    uint32_t ksc[2] = {0u, 0u};
    if constexpr (MX) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) ksc[kt] = mx_lane_scales(__float_as_uint(kls[cur][32 * kt + nn]), hh);
    }
    float p[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v16f acc = {};
        if constexpr (MX) {
          acc = mfma_mx<0>(qa[mt][0], kb[kt][0], acc, qsc[mt], ksc[kt]);
          acc = mfma_mx<1>(qa[mt][1], kb[kt][1], acc, qsc[mt], ksc[kt]);
        } else {
          acc = mfma_f8(qa[mt][0], kb[kt][0], acc);
          acc = mfma_f8(qa[mt][1], kb[kt][1], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sum = fmaf(wr[mt][r], __int_as_float(max(__float_as_int(acc[r]), 0)), sum);
      }
      p[kt] = sum;
    }
    // lane l < 32 holds half of the heads of keys l (p[0]) and 32+l (p[1]),
    // lane 32+l the other half: swap the cross halves, then one add gives lane
    // l the score of key l
    const auto hv = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
    float score = __uint_as_float(hv[0]) + __uint_as_float(hv[1]);
    if constexpr (!MX) score *= ks;
    const int lim = pos - 64 * c;  // keys of this page up to offset lim are visible
    if (lim < 63) score = lane > lim ? -INFINITY : score;
    // a descriptor over the row from this page on, ending at max_visible: its
    // range check drops the stores past the row's end
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(srow + 64 * c, 0, (a.s.max_visible - 64 * c) * 4, kRawBuffer);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), prs, lane * 4, 0, 0);
  };

  for (int i = 0; i < nq; ++i) {
    int b = -1;
#pragma unroll
    for (int j = 0; j < kSQ; ++j) b = j == i ? qseq[j] : b;
    b = __builtin_amdgcn_readfirstlane(b);
    bool seen = false;
    int ce = 0;
#pragma unroll
    for (int j = 0; j < kSQ; ++j) {
      seen = seen || (j < i && qseq[j] == b);
      ce = qseq[j] == b ? max(ce, cvis[j]) : ce;
    }
    if (seen) continue;
    const int c_end = min(c_begin + kSChunk, __builtin_amdgcn_readfirstlane(ce));
    if (c_begin >= c_end) continue;
    const bool mine = my_seq == b;

    // key pages: global -> registers (two pages ahead) -> LDS (double buffer);
    // lane l of pg[k] holds the physical page of chunk page 64k + l
    const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;
    constexpr int NPG = kSChunk / 64;
    int pg[NPG];
#pragma unroll
    for (int k = 0; k < NPG; ++k) pg[k] = clampi(table[min(c_begin + 64 * k + lane, c_end - 1)], 0, a.s.num_pages - 1);
    auto gload = [&](int c) __attribute__((always_inline)) {
      const int o = min(c, c_end - 1) - c_begin;
      int sel = pg[0];
#pragma unroll
      for (int k = 1; k < NPG; ++k) sel = (o >> 6) == k ? pg[k] : sel;
      const int page = __builtin_amdgcn_readlane(sel, o & 63);
      const __amdgpu_buffer_rsrc_t krs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kpool + (int64_t)page * (kPage * 128)), 0, kPage * 128, kRawBuffer);
      // every wave loads the scales, wave 0 stores them: fp8 the key scale,
      // MX the key's four group-scale bytes (as raw bits)
      const void* sbase = MX ? (const void*)(a.k_mx + (int64_t)page * kPage * 4) : (const void*)(a.k_scale + (int64_t)page * kPage);
      const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, 0, kPage * 4, kRawBuffer);
      KStage g;
      const v4i x = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(krs, kvoff, 0, 0));
      const v4i y = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(krs, kvoff + 16, 0, 0));
      g.x = make_uint4(x[0], x[1], x[2], x[3]);
      g.y = make_uint4(y[0], y[1], y[2], y[3]);
      g.s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksr, lane * 4, 0, 0));
      return g;
    };
    auto lwrite = [&](int buf, const KStage& g) __attribute__((always_inline)) {
      *(uint4*)&kl[buf][kswz(sr, sj)] = g.x;
      *(uint4*)&kl[buf][kswz(sr, sj + 1)] = g.y;
      if (wave == 0) kls[buf][lane] = g.s;
    };
    // at step c: page c is in LDS buffer c & 1, page c+1 in one register
    // stage, page c+2 in flight into the other
    KStage sa = gload(c_begin), sb = gload(c_begin + 1);
    __syncthreads();  // the previous round's reads of both buffers are done
    lwrite(0, sa);
    sa = gload(c_begin + 2);
    int c = c_begin;
    for (; c + 2 <= c_end; c += 2) {
      __syncthreads();
      lwrite(1, sb);
      sb = gload(c + 3);
      if (mine && c < c_own) compute(c, 0);
      __syncthreads();
      lwrite(0, sa);
      sa = gload(c + 4);
      if (mine && c + 1 < c_own) compute(c + 1, 1);
    }
    if (c < c_end) {
      __syncthreads();
      if (mine && c < c_own) compute(c, 0);
    }
  }
}

hipError_t launch_index_scores(const sia_indexer_in& in, const SeqArgs& s, float* scores, int64_t ld,
                               hipStream_t st) {
  const IndexArgs a = index_args(in, s, scores, ld);
  if (s.T == 0 || s.max_visible == 0) return hipSuccess;
  const bool mx = in.dtype == SIA_MXFP8_E4M3;
  if (in.dtype == SIA_BF16) return launch_index_scores_bf16(in, s, scores, ld, st);
  if (in.dtype == SIA_F32) {
    dim3 grid(s.T, (s.max_visible + 255) / 256);
    hipLaunchKernelGGL(k_index_scores_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int n_chunks = (s.max_visible + 63) / 64;
  if (s.T >= kSQ * s.batch && s.max_visible <= (1 << 29)) {
    // several queries per sequence on average: share key pages across queries
    const int nqb = (s.T + kSQ - 1) / kSQ;
    const int64_t grid = (int64_t)nqb * ((n_chunks + kSChunk - 1) / kSChunk);
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), blk(kSThreads);
    if (in.heads == 64) {
      if (mx)
        hipLaunchKernelGGL((k_index_scores_fp8_shared<64, true>), g, blk, 0, st, a, nqb);
      else
        hipLaunchKernelGGL((k_index_scores_fp8_shared<64, false>), g, blk, 0, st, a, nqb);
    } else {
      if (mx)
        hipLaunchKernelGGL((k_index_scores_fp8_shared<32, true>), g, blk, 0, st, a, nqb);
      else
        hipLaunchKernelGGL((k_index_scores_fp8_shared<32, false>), g, blk, 0, st, a, nqb);
    }
    return hipGetLastError();
  }
  const int n_qblocks = (s.T + 3) / 4;
  // enough waves to keep every CU busy: split the key range of each query
  // block when there are few query blocks (decode), keep it whole otherwise
  const int cus = num_cus();
  const int64_t target_items = (int64_t)cus * 2;
  int n_ranges = (int)((target_items + n_qblocks - 1) / n_qblocks);
  // at most 64 pages per item: a wave holds its item's page ids one per lane
  n_ranges = max(n_ranges, (n_chunks + 63) / 64);
  n_ranges = n_ranges < 1 ? 1 : (n_ranges > n_chunks ? n_chunks : n_ranges);
  const int cpi = (n_chunks + n_ranges - 1) / n_ranges;
  const int64_t items = (int64_t)n_qblocks * ((n_chunks + cpi - 1) / cpi);
  const int64_t resident = (int64_t)cus * 2;
  const int grid = (int)(items < resident ? items : resident);
  if (in.heads == 64) {
    if (mx)
      hipLaunchKernelGGL((k_index_scores_fp8<64, true>), dim3(grid), dim3(256), 0, st, a, n_qblocks, n_chunks, cpi);
    else
      hipLaunchKernelGGL((k_index_scores_fp8<64, false>), dim3(grid), dim3(256), 0, st, a, n_qblocks, n_chunks, cpi);
  } else {
    if (mx)
      hipLaunchKernelGGL((k_index_scores_fp8<32, true>), dim3(grid), dim3(256), 0, st, a, n_qblocks, n_chunks, cpi);
    else
      hipLaunchKernelGGL((k_index_scores_fp8<32, false>), dim3(grid), dim3(256), 0, st, a, n_qblocks, n_chunks, cpi);
  }
  return hipGetLastError();
}

}  // namespace sia

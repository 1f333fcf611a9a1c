// Step 2, block-aligned form — selection of whole cache pages.
//
// [P3] "Day-One Inference Adaptation for Very Large Hybrid-Attention Models:
//      From Operators to Serving Systems", section 3.1: the selection result is
//      aligned to cache blocks so that attention reads the cache in whole blocks.
//
// A page (64 consecutive positions, the cache block) is ranked by the largest
// score among its visible positions.  The first K/64 pages under (page score
// desc, page asc) are kept, and every visible position of a kept page is
// emitted, pages in ascending order, -1 padding up to K.  Three launches:
//  1. k_page_max: per row, the maximum of each visible page (16 lanes x float4
//     per page, combined with a DPP max inside the 16-lane row) and the index
//     of the row's last visible page;
//  2. the per-query Top-K (k_topk, ascending order) over the page scores with
//     K/64 entries;
//  3. k_expand_pages: kept page ids -> positions (and, optionally, each
//     position's page score).
#include "block_prims.hpp"
#include "sia_internal.hpp"

namespace sia {

namespace {

constexpr int kPMThreads = 256;
constexpr int kPMPages = 64;  // pages per workgroup: four rounds of 16 pages
constexpr int kEXThreads = 256;

__device__ __forceinline__ int visible(const SeqArgs& s, int t, int64_t lim) {
  return clampi(s.q_pos[t], -1, (int)lim - 1) + 1;
}

__global__ __launch_bounds__(kPMThreads) void k_page_max(const float* __restrict__ scores, int64_t ld, SeqArgs s,
                                                         int64_t lim, int chunks, float* __restrict__ pscore,
                                                         int64_t ldp, int32_t* __restrict__ plast) {
  const int t = (int)(blockIdx.x / (unsigned)chunks);
  const int c = (int)(blockIdx.x % (unsigned)chunks);
  const int n = visible(s, t, lim);
  if (c == 0 && threadIdx.x == 0) plast[t] = n > 0 ? (n - 1) >> 6 : -1;
  const int sub = threadIdx.x & 15;
  const float* row = scores + (int64_t)t * ld;
  // The four rounds' loads are unconditional and issued together: this
  // workgroup's part of the row goes through a buffer descriptor that ends at
  // the first group of four past the row's visible entries (lim rounded up to
  // 4 is still inside the row, ld being a multiple of 4), loads past it
  // return zeros, and positions at or past n are masked to key 0 afterwards.
  // A conditional load per round cost one memory latency each.
  const int64_t x0 = (int64_t)c * kPMPages * kPage;  // first position of this workgroup's pages
  int64_t span = ((lim + 3) & ~(int64_t)3) - x0;
  span = span < 0 ? 0 : (span > kPMPages * kPage ? kPMPages * kPage : span);
  const __amdgpu_buffer_rsrc_t rrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(row + x0), 0, (int)(span * 4), kRawBuffer);
  v4i v[kPMPages / 16];
#pragma unroll
  for (int r = 0; r < kPMPages / 16; ++r) {
    const int lp = r * 16 + (int)(threadIdx.x >> 4);   // page within the workgroup's 64
    v[r] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rrs, (lp * kPage + sub * 4) * 4, 0, 0));
  }
#pragma unroll
  for (int r = 0; r < kPMPages / 16; ++r) {
    const int p = c * kPMPages + r * 16 + (int)(threadIdx.x >> 4);
    const int x = p * kPage + sub * 4;
    uint32_t k = 0u;  // below every float's key
#pragma unroll
    for (int q = 0; q < 4; ++q) k = max(k, f2key(__int_as_float(v[r][q])) & (uint32_t)((x + q - n) >> 31));
    k = row_incl(k, 0u, OpMax{});  // lane 15 of each 16-lane row: the page maximum
    if (sub == 15 && p * kPage < n) pscore[(int64_t)t * ldp + p] = key2f(k);
  }
}

// Four consecutive outputs per thread (K is a multiple of 64, so they share a page).
__global__ __launch_bounds__(kEXThreads) void k_expand_pages(const int32_t* __restrict__ pidx,
                                                             const float* __restrict__ pval, int kp, SeqArgs s,
                                                             int64_t lim, int K, int64_t total,
                                                             int32_t* __restrict__ idx, float* __restrict__ vals) {
  const int64_t e = ((int64_t)blockIdx.x * kEXThreads + threadIdx.x) * 4;
  if (e >= total) return;
  const int t = (int)(e / K);
  const int j = (int)(e - (int64_t)t * K);
  const int slot = j >> 6;
  const int page = pidx[(int64_t)t * kp + slot];
  const int n = visible(s, t, lim);
  const int base = page * kPage + (j & (kPage - 1));
  const float pv = (vals && page >= 0) ? pval[(int64_t)t * kp + slot] : -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool ok = page >= 0 && base + u < n;
    idx[e + u] = ok ? base + u : -1;
    if (vals) vals[e + u] = ok ? pv : -INFINITY;
  }
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int64_t topk_pages_ld(int max_visible) { return ((int64_t)(max_visible + kPage - 1) / kPage + 3) / 4 * 4; }

size_t topk_pages_ws_bytes(int T, int max_visible, int K) {
  const size_t kp = (size_t)(K / kPage);
  return a256((size_t)T * topk_pages_ld(max_visible) * sizeof(float)) + a256((size_t)T * sizeof(int32_t)) +
         2 * a256((size_t)T * kp * sizeof(int32_t));
}

hipError_t launch_topk_pages(const float* scores, int64_t ld, const SeqArgs& s, int K, int32_t* idx, float* vals,
                             void* ws, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (K < kPage || K % kPage != 0) return hipErrorInvalidValue;
  const int kp = K / kPage;
  const int64_t lim = ld < (int64_t)s.max_visible ? ld : (int64_t)s.max_visible;
  const int64_t ldp = topk_pages_ld(s.max_visible);
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* pscore = reinterpret_cast<float*>(w);
  w += a256((size_t)s.T * ldp * sizeof(float));
  int32_t* plast = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)s.T * sizeof(int32_t));
  int32_t* pidx = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)s.T * kp * sizeof(int32_t));
  float* pval = reinterpret_cast<float*>(w);

  const int pages = (int)((lim + kPage - 1) / kPage);
  const int chunks = (pages + kPMPages - 1) / kPMPages;
  const int64_t grid1 = (int64_t)s.T * chunks;
  const int64_t total = (int64_t)s.T * K;
  const int64_t grid3 = (total / 4 + kEXThreads - 1) / kEXThreads;
  if (grid1 > 0x7fffffff || grid3 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_page_max, dim3((unsigned)grid1), dim3(kPMThreads), 0, st, scores, ld, s, lim, chunks, pscore,
                     ldp, plast);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  SeqArgs sp = s;  // the same rows over page scores: visible pages 0..plast[t]
  sp.q_pos = plast;
  sp.max_visible = pages;
  e = launch_topk(pscore, ldp, sp, kp, 1, pidx, vals ? pval : nullptr, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_expand_pages, dim3((unsigned)grid3), dim3(kEXThreads), 0, st, pidx, pval, kp, s, lim, K,
                     total, idx, vals);
  return hipGetLastError();
}

}  // namespace sia

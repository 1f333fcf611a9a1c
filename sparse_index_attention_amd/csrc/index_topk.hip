// Steps 1 and 2 fused — indexer scores and per-query Top-K without a score
// matrix in memory.
//
// [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models",
//      section "Sparse Attention Pipeline Optimization": scoring, head-weight
//      summation and Top-K selection as one operator that reads the paged K cache
//      and never writes the score matrix back.
// [P4] "Inference Acceleration for New LLM Architectures", section 2: the fused
//      operator keeps scores in registers or shared memory and emits only the
//      selected index list.
// [P5] "Inference Adaptation and Performance Optimization for a Domestically
//      Developed LLM's New Architecture", section 3.1: LI fusion.
//
// Pass 1 (k_index_topk_ranges): one workgroup = one query x one range of 128
// pages (8192 keys).  Its eight waves score 16 pages each into LDS; the
// workgroup then keeps the range's first min(K, keys) entries under (score
// desc, position asc) — an exact radix select for the threshold key and an
// ordered pass for ties — and writes them in ascending position order to the
// query's candidate list, slots [r*K, r*K + count).  Every range before the
// last holds 8192 >= K keys and contributes exactly K entries, so the list is
// contiguous.
// Pass 2 is the Top-K kernel on each query's candidate list with a map back to
// positions.  A member of the query's Top-K is a member of its range's Top-K,
// so selecting from the candidates gives the same set; the list is in
// ascending position order, so ties still resolve toward lower positions.
#include "block_prims.hpp"
#include "index_core.hpp"

namespace sia {

constexpr int kRangePages = kIndexTopkRangeKeys / kPage;  // 128
constexpr int kRNT = 512;
constexpr int kRNW = kRNT / 64;
constexpr int kRPer = kIndexTopkRangeKeys / kRNT;          // keys per thread: 16
constexpr int kRBins = 2048;
constexpr int kRList = kRNT;
static_assert(2 * kMaxTopK <= kIndexTopkRangeKeys, "output staging reuses the score buffer");  // threshold-bin keys ranked by brute force (one per thread)

struct RangeSmem {
  float sc[kIndexTopkRangeKeys];  // scores; after the keys are in registers, the output staging
  uint32_t hist[kRBins];
  uint32_t lkey[kRList];
  int32_t lpos[kRList];
  uint32_t red[2][kRNW];
  uint32_t scan[2][kRNW];
  uint32_t found_bin, found_above, found_cnt, list_n, found_key, found_need;
  uint32_t next_page;  // pages of the range claimed so far
  int32_t pages[kRangePages];  // physical pages of the range
};

template <int HI, bool MX>
__global__ __launch_bounds__(kRNT, 1) void k_index_topk_ranges(IndexArgs a, int K, int n_ranges,
                                                               float* __restrict__ cscore,
                                                               int32_t* __restrict__ cpos, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) RangeSmem sh;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index();
  // longest rows first when positions grow with t
  const int item = (int)blockIdx.x;
  const int t = a.s.T - 1 - item / n_ranges;
  const int r = item % n_ranges;
  const int pos = clampi(a.s.q_pos[t], -1, a.s.max_visible - 1);
  const int n = pos + 1;
  const int c_vis = n > 0 ? (pos >> 6) + 1 : 0;
  const int c0 = r * kRangePages;
  if (c0 >= c_vis) return;
  const int c1 = c0 + kRangePages < c_vis ? c0 + kRangePages : c_vis;
  const int key0 = r * kIndexTopkRangeKeys;
  const int nr = n - key0 < kIndexTopkRangeKeys ? n - key0 : kIndexTopkRangeKeys;
  const int b = clampi(a.s.q_seq[t], 0, a.s.batch - 1);

  // ---- 1. scores of the range into LDS.  The waves claim pages one at a
  // time from a shared counter: with a fixed share each, the slowest wave's
  // memory latency would hold up the whole workgroup at the barrier.
  // The range's block-table entries go to LDS first, so that the page loop
  // looks them up without a memory load.
  // The first histogram pass's bins are cleared here as well, and each lane
  // tracks the key range of the scores it writes, so that the selection
  // starts right after the scoring barrier.
  if (tid == 0) {
    sh.next_page = 0;
    sh.list_n = 0;
  }
  if (tid < kRangePages) sh.pages[tid] = a.s.block_table[(int64_t)b * a.s.max_pages + min(c0 + tid, c1 - 1)];
  for (int i = tid; i < kRBins; i += kRNT) sh.hist[i] = 0;
  uint32_t lmn = 0xffffffffu, lmx = 0u;
  __syncthreads();
  score_claimed_pages<HI, MX>(
      a, t, pos,
      [&]() __attribute__((always_inline)) -> int {
        uint32_t v = 0;
        if (lane == 0) v = atomicAdd(&sh.next_page, 1u);
        const int c = c0 + __builtin_amdgcn_readfirstlane((int)v);
        return c < c1 ? c : -1;
      },
      [&](int c) __attribute__((always_inline)) { return sh.pages[c < c0 ? 0 : c - c0]; },
      [&](int s, float score) __attribute__((always_inline)) {
        sh.sc[s - key0] = score;
        const uint32_t k = s <= pos ? f2key(score) : 0u;  // 0: past the range's keys
        lmn = k && k < lmn ? k : lmn;
        lmx = k > lmx ? k : lmx;
      });
  lmn = wave_all(lmn, 0xffffffffu, OpMin{});
  lmx = wave_all(lmx, 0u, OpMax{});
  if (lane == 0) {
    sh.red[0][w] = lmn;
    sh.red[1][w] = lmx;
  }
  __syncthreads();

  // ---- 2. keys in registers: thread tid holds positions 16*tid .. 16*tid+15
  uint32_t key[kRPer];
  {
    const float4* src = reinterpret_cast<const float4*>(sh.sc) + (kRPer / 4) * tid;
#pragma unroll
    for (int q = 0; q < kRPer / 4; ++q) {
      const float4 v = src[q];
      const int p = kRPer * tid + 4 * q;
      key[4 * q] = p < nr ? f2key(v.x) : 0u;  // 0: past the range's keys
      key[4 * q + 1] = p + 1 < nr ? f2key(v.y) : 0u;
      key[4 * q + 2] = p + 2 < nr ? f2key(v.z) : 0u;
      key[4 * q + 3] = p + 3 < nr ? f2key(v.w) : 0u;
    }
  }
  const int cnt = nr < K ? nr : K;

  // threshold key T and the number `need` of keys equal to T to keep (lowest
  // positions first); with nr <= K every key is kept
  uint32_t T = 0u, need = 0u;
  int pp = 0;
  if (nr > K) {
    const uint32_t kmn = waves_all<kRNW>(sh.red[0], 0xffffffffu, OpMin{});
    const uint32_t kmx = waves_all<kRNW>(sh.red[1], 0u, OpMax{});
    uint32_t lo = kmn;
    uint64_t range = kmx >= kmn ? (uint64_t)kmx - kmn + 1 : 1;
    need = (uint32_t)K;
    bool ranked = false, first = true;
    // Each pass narrows [lo, lo + range) to the bin holding the need-th
    // largest remaining key.  Once that bin holds at most kRList keys, they
    // are ranked directly under (key desc, position asc) instead.
    while (range > 1) {
      const int shift = bin_shift(range);
      const int nb = (int)((range - 1) >> shift) + 1;
      if (!first) {  // the first pass's bins were cleared before the scores
        for (int i = tid; i < kRBins; i += kRNT) sh.hist[i] = 0;
        if (tid == 0) sh.list_n = 0;
        __syncthreads();
      }
      first = false;
#pragma unroll
      for (int j = 0; j < kRPer; ++j) {
        const uint32_t k = key[j];
        if (k && k >= lo && (uint64_t)(k - lo) < range) atomicAdd(&sh.hist[(k - lo) >> shift], 1u);
      }
      __syncthreads();
      // thread tid owns bins hb .. hb - 3, counted from the top
      const int hb = kRBins - 1 - 4 * tid;
      uint32_t cb[4], csum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cb[q] = hb - q < nb ? sh.hist[hb - q] : 0u;
        csum += cb[q];
      }
      uint32_t tot;
      uint32_t above = block_excl<kRNW>(csum, sh.scan[pp], tot);
      pp ^= 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < need && need <= above + cb[q]) {
          sh.found_bin = (uint32_t)(hb - q);
          sh.found_above = above;
          sh.found_cnt = cb[q];
        }
        above += cb[q];
      }
      __syncthreads();
      const uint32_t bsel = sh.found_bin, above_sel = sh.found_above, in_bin = sh.found_cnt;
      __syncthreads();
      need -= above_sel;
      const uint64_t off = (uint64_t)bsel << shift;
      lo = lo + (uint32_t)off;
      const uint64_t rest = range - off;
      const uint64_t width = (uint64_t)1 << shift;
      range = rest < width ? rest : width;
      if (range > 1 && in_bin <= (uint32_t)kRList) {
        // the in_bin keys of [lo, lo + range): the need-th of them under
        // (key desc, position asc) is the last one kept
#pragma unroll
        for (int j = 0; j < kRPer; ++j) {
          const uint32_t k = key[j];
          if (k && k >= lo && (uint64_t)(k - lo) < range) {
            const uint32_t slot = atomicAdd(&sh.list_n, 1u);
            sh.lkey[slot] = k;
            sh.lpos[slot] = kRPer * tid + j;
          }
        }
        __syncthreads();
        if (tid < (int)in_bin) {
          const uint32_t mk = sh.lkey[tid];
          const int mp = sh.lpos[tid];
          const uint64_t mine = composite(mk, mp);
          uint32_t rank = 0, eq_upto = 0;
          for (int i = 0; i < (int)in_bin; ++i) {
            const uint32_t k = sh.lkey[i];
            const int p = sh.lpos[i];
            rank += composite(k, p) < mine;
            eq_upto += k == mk && p <= mp;
          }
          if (rank == need - 1) {
            sh.found_key = mk;
            sh.found_need = eq_upto;
          }
        }
        __syncthreads();
        T = sh.found_key;
        need = sh.found_need;
        ranked = true;
        break;
      }
    }
    if (!ranked) T = lo;
  }

  // ---- 3. ordered pass: keys > T, then the first `need` keys == T, staged in
  // LDS in position order and written out coalesced
  uint32_t cgt = 0, ceq = 0;
#pragma unroll
  for (int j = 0; j < kRPer; ++j) {
    cgt += key[j] > T;
    ceq += key[j] != 0u && key[j] == T && need > 0;
  }
  uint32_t tot;
  const uint32_t pre = block_excl<kRNW>(cgt | (ceq << 16), sh.scan[pp], tot);
  uint32_t g = pre & 0xffffu, e = pre >> 16;
  float* stage_val = sh.sc;                                          // [K]
  int32_t* stage_pos = reinterpret_cast<int32_t*>(sh.sc + kMaxTopK);  // [K]
#pragma unroll
  for (int j = 0; j < kRPer; ++j) {
    const uint32_t k = key[j];
    const bool gt = k > T;
    const bool eq = k != 0u && k == T && need > 0;
    if (gt || (eq && e < need)) {
      const uint32_t slot = g + (e < need ? e : need);
      if ((int)slot < cnt) {
        stage_val[slot] = key2f(k);
        stage_pos[slot] = key0 + kRPer * tid + j;
      }
    }
    g += gt;
    e += eq;
  }
  __syncthreads();
  float* crow = cscore + (int64_t)t * ldc + (int64_t)r * K;
  int32_t* prow = cpos + (int64_t)t * ldc + (int64_t)r * K;
  for (int i = tid; i < cnt; i += kRNT) {
    crow[i] = stage_val[i];
    prow[i] = stage_pos[i];
  }
}

int index_topk_ranges(int max_visible) {
  return (max_visible + kIndexTopkRangeKeys - 1) / kIndexTopkRangeKeys;
}

int64_t index_topk_ld(int max_visible, int K) {
  return ((int64_t)index_topk_ranges(max_visible) * K + 3) / 4 * 4;
}

hipError_t launch_index_topk(const sia_indexer_in& in, const SeqArgs& s, int K, int order, int32_t* idx,
                             float* vals, float* cscore, int32_t* cpos, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const IndexArgs a = index_args(in, s, nullptr, 0);
  const bool mx = in.dtype == SIA_MXFP8_E4M3;
  const int n_ranges = index_topk_ranges(s.max_visible);
  const int64_t ldc = index_topk_ld(s.max_visible, K);
  if (n_ranges > 0) {
    const dim3 grid((unsigned)((int64_t)s.T * n_ranges));
    if (in.heads == 64) {
      if (mx)
        hipLaunchKernelGGL((k_index_topk_ranges<64, true>), grid, dim3(kRNT), 0, st, a, K, n_ranges, cscore, cpos, ldc);
      else
        hipLaunchKernelGGL((k_index_topk_ranges<64, false>), grid, dim3(kRNT), 0, st, a, K, n_ranges, cscore, cpos, ldc);
    } else {
      if (mx)
        hipLaunchKernelGGL((k_index_topk_ranges<32, true>), grid, dim3(kRNT), 0, st, a, K, n_ranges, cscore, cpos, ldc);
      else
        hipLaunchKernelGGL((k_index_topk_ranges<32, false>), grid, dim3(kRNT), 0, st, a, K, n_ranges, cscore, cpos, ldc);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_topk_candidates(cscore, cpos, ldc, kIndexTopkRangeKeys, s, K, order, idx, vals, st);
}

}  // namespace sia

// Step 2 — per-query Top-K over the visible scores.
//
// [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models",
//      section "Sparse Attention Pipeline Optimization": keep the K best-scored
//      history positions of each query.
// [P2] "Efficient Inference Deployment and Optimization for Hybrid Attention
//      LLMs", section 3.2: Top-K consumes the index scores.
//
// Selected set: the first min(K, n) positions under (score desc, position asc),
// with -0 == +0.  One 1024-thread workgroup per query row.  Scores are mapped to
// order-preserving 32-bit keys; (key desc, position asc) is the ascending order
// of the 64-bit composite (~key << 32 | position), which is unique per row.
//
// Fast path (keys held in registers when the row fits, else streamed):
//  1. Block-wide key range [kmin, kmax].  Rows longer than kDirect also take one
//     key sample per thread and place a lower bound L on the K-th key: the
//     sample histogram over [kmin, kmax] gives the bin that holds the r-th
//     largest sample, r sized so that the keys >= L outnumber K with a wide
//     margin.  Shorter rows use L = kmin.
//  2. Histogram of the keys >= L (a few thousand LDS atomics instead of one
//     per key) over 2048 equal-width bins of [L, kmax].  A suffix scan gives
//     each bin's start in the output order and the bin b* holding the last
//     selected key.
//  3. Keys in bins >= b* are scattered into their bins; each one's rank inside
//     its bin (a short brute-force count over the composite) gives its final
//     place.  Order 0 writes it there directly; order 1 sets a position bitmap
//     and compacts it in position order.
// The fast path is exact whenever it completes.  It hands the row to the exact
// radix path below when its assumptions fail (fewer than K keys >= L, a bin
// with more than kMaxBin entries, e.g. long runs of equal scores).
//
// Exact path: range-adaptive radix select (<= 2048 bins per pass, three passes
// close a 32-bit range), an ordered pass that keeps every key above the
// threshold and the lowest-position ties, and a bitonic sort for order 0.
#include "block_prims.hpp"
#include "sia_internal.hpp"

namespace sia {

constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;
constexpr int kBins = 2048;
constexpr int kMaxK = 2048;
constexpr int kMaxBin = 256;
constexpr int kBuf = kMaxK + kMaxBin;
constexpr int kStreamWords = 8192;  // order-1 bitmap of streamed rows: 262144 positions
constexpr int kDirect = 8192;  // rows up to this long histogram every key (no sample bound)
constexpr int kStreamLoads = 8;     // loads in flight per thread in a streamed pass

// ---- exact path ----------------------------------------------------------------
struct ExactSmem {
  uint32_t hist[kBins];
  uint64_t sel[kMaxK];
  uint32_t red[2][kNW];
  uint32_t scan[2][kNW];
  uint32_t found_bin, found_above;
};

// Writes out[0 .. min(K, n)) for one row, reading the scores from memory.
__device__ __noinline__ void topk_exact(const float* __restrict__ row, int n, int K, int order,
                                        int32_t* __restrict__ orow, float* __restrict__ vrow,
                                        const int32_t* __restrict__ pmap, ExactSmem& sh) {
  __syncthreads();  // every thread is done with the fast path's shared state
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index();
  int pp = 0;  // ping-pong between the two scan slots

  // 1. key range
  uint32_t T = 0u, need = 0u;
  if (n > K) {
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    for (int i = tid; i < n; i += kNT) {
      const uint32_t k = f2key(row[i]);
      kmn = min(kmn, k);
      kmx = max(kmx, k);
    }
    kmn = wave_all(kmn, 0xffffffffu, OpMin{});
    kmx = wave_all(kmx, 0u, OpMax{});
    if (lane == 0) {
      sh.red[0][w] = kmn;
      sh.red[1][w] = kmx;
    }
    __syncthreads();
    kmn = waves_all<kNW>(sh.red[0], 0xffffffffu, OpMin{});
    kmx = waves_all<kNW>(sh.red[1], 0u, OpMax{});

    // 2. threshold key: narrow [lo, lo + range) to the bin holding the K-th key
    uint32_t lo = kmn;
    uint64_t range = (uint64_t)kmx - kmn + 1;
    need = (uint32_t)K;
    while (range > 1) {
      const int shift = bin_shift(range);
      const int nb = (int)((range - 1) >> shift) + 1;
      for (int i = tid; i < kBins; i += kNT) sh.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kNT) {
        const uint32_t k = f2key(row[i]);
        if (k >= lo && (uint64_t)(k - lo) < range) atomicAdd(&sh.hist[(k - lo) >> shift], 1u);
      }
      __syncthreads();
      // thread t owns bins hb and hb - 1, counted from the top
      const int hb = kBins - 1 - 2 * tid;
      const uint32_t c0 = hb < nb ? sh.hist[hb] : 0u, c1 = hb - 1 < nb ? sh.hist[hb - 1] : 0u;
      uint32_t tot;
      const uint32_t a0 = block_excl<kNW>(c0 + c1, sh.scan[pp], tot);
      pp ^= 1;
      const uint32_t a1 = a0 + c0;
      if (a0 < need && need <= a0 + c0) {
        sh.found_bin = (uint32_t)hb;
        sh.found_above = a0;
      }
      if (a1 < need && need <= a1 + c1) {
        sh.found_bin = (uint32_t)(hb - 1);
        sh.found_above = a1;
      }
      __syncthreads();
      const uint32_t bsel = sh.found_bin, above_sel = sh.found_above;
      __syncthreads();
      need -= above_sel;
      const uint64_t off = (uint64_t)bsel << shift;
      lo = lo + (uint32_t)off;
      const uint64_t rest = range - off;
      const uint64_t width = (uint64_t)1 << shift;
      range = rest < width ? rest : width;
    }
    T = lo;
  }

  // 3. ordered selection: keys > T, then the lowest positions among keys == T
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += kNT * 4) {
    uint32_t kk[4];
    uint32_t cnt_gt = 0, cnt_eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + tid * 4 + j;
      kk[j] = i < n ? f2key(row[i]) : 0u;
      cnt_gt += (i < n) && kk[j] > T;
      cnt_eq += (i < n) && kk[j] == T && need > 0;
    }
    uint32_t tot;
    const uint32_t pre = block_excl<kNW>(cnt_gt | (cnt_eq << 16), sh.scan[pp], tot);
    pp ^= 1;
    uint32_t g = run_gt + (pre & 0xffffu), e = run_eq + (pre >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + tid * 4 + j;
      const bool gt = (i < n) && kk[j] > T;
      const bool eq = (i < n) && kk[j] == T && need > 0;
      if (gt || (eq && e < need)) {
        const uint32_t slot = g + (e < need ? e : need);
        sh.sel[slot] = composite(kk[j], i);
      }
      g += gt;
      e += eq;
    }
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
  __syncthreads();

  // 4. output
  const int cnt = n < K ? n : K;
  if (order == 0 && cnt > 1) {
    int P = 1;
    while (P < cnt) P <<= 1;
    for (int i = cnt + tid; i < P; i += kNT) sh.sel[i] = ~0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P / 2; i += kNT) {
          const int a = (i / j) * 2 * j + (i % j);
          const int bb = a + j;
          const uint64_t x = sh.sel[a], y = sh.sel[bb];
          const bool up = (a & k) == 0;
          if ((x > y) == up) {
            sh.sel[a] = y;
            sh.sel[bb] = x;
          }
        }
        __syncthreads();
      }
    }
  }
  // order 1 keeps the selection pass's ascending position order
  for (int i = tid; i < cnt; i += kNT) {
    const uint64_t v = sh.sel[i];
    const int p = (int)(uint32_t)v;
    orow[i] = pmap ? pmap[p] : p;
    if (vrow) vrow[i] = key2f(~(uint32_t)(v >> 32));
  }
}

// ---- fast path -------------------------------------------------------------------
template <int PER>
struct FastSmem {
  static constexpr int kWords = PER > 0 ? kNT * PER / 32 : kStreamWords;
  uint32_t hs[kBins];     // sample histogram
  uint32_t hist[kBins];   // histogram of the keys >= L
  uint32_t above[kBins];  // keys in higher bins = the bin's first output slot
  uint32_t cur[kBins];    // fill cursors
  uint64_t buf[kBuf];     // composites of bins >= b*, grouped by bin
  uint32_t bitmap[kWords];
  uint32_t red[3][kNW];
  uint32_t scan[3][kNW];
  uint32_t maxm[kNW];
  uint32_t L, bstar, estar;
};
template <int PER>
union TopkSmem {
  FastSmem<PER> f;
  ExactSmem x;
};

// threadIdx.x through an opaque move: positions derived from it are then
// recomputed in each pass over the keys instead of being kept in sixty-four
// registers across the passes.
__device__ __forceinline__ int opaque_tid() {
  int x;
  asm volatile("v_mov_b32 %0, %1" : "=v"(x) : "v"((int)threadIdx.x));
  return x;
}

// Calls f(key, position, slot) for every position of the row this thread
// covers; key 0 marks a position past the row's end.  Position of register
// slot 4j + q: (j * kNT + tid) * 4 + q (streamed rows: the same with j
// counting the groups of four from the row's start, and slot -1).
template <int PER, typename F>
__device__ __forceinline__ void for_keys(const uint32_t (&key)[PER > 0 ? PER : 1], const float* __restrict__ row,
                                         int n, F&& f) {
  if constexpr (PER > 0) {
    const int tid = opaque_tid();
#pragma unroll
    for (int j = 0; j < PER / 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) f(key[4 * j + q], (j * kNT + tid) * 4 + q, 4 * j + q);
  } else {
    // streamed: kStreamLoads loads of four keys per thread are issued together
    // (one memory latency per 32 768 keys, not per 4 096); the descriptor's
    // range ends at the last whole group of four holding a visible key, and
    // loads past it return zeros without a memory access
    const __amdgpu_buffer_rsrc_t rrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, ((n + 3) & ~3) * 4, kRawBuffer);
    const int tid = opaque_tid();
    for (int base = 0; base < n; base += kNT * 4 * kStreamLoads) {
      v4i v[kStreamLoads];
#pragma unroll
      for (int u = 0; u < kStreamLoads; ++u)
        v[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rrs, tid * 16, (base + u * kNT * 4) * 4, 0));
#pragma unroll
      for (int u = 0; u < kStreamLoads; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = base + (u * kNT + tid) * 4 + q;
          f(f2key(__int_as_float(v[u][q])) & (uint32_t)((p - n) >> 31), p, -1);
        }
    }
  }
}

// PER keys per thread live in registers (rows up to kNT * PER); PER = 0 streams
// the row from memory on every pass.  CAND: the rows are candidate lists with a
// map back to positions; with PER <= 32 each thread also holds the positions
// of its keys, so that score-order output needs no dependent load of the map.
// Rows of n keys with n_lo < n <= n_hi are this launch's; the others belong to
// another launch (another PER) and their workgroups return at once.
template <int PER, bool CAND>
__global__ __launch_bounds__(kNT) void k_topk(const float* __restrict__ scores, int64_t ld, SeqArgs s, int K,
                                              int order, int32_t* __restrict__ idx, float* __restrict__ vals,
                                              CandMap cm, int n_lo, int n_hi) {
  constexpr bool kCarry = CAND && PER > 0 && PER <= 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  TopkSmem<PER>& smem = *reinterpret_cast<TopkSmem<PER>*>(smem_raw);
  FastSmem<PER>& sh = smem.f;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_index();
  const int t = s.T - 1 - (int)blockIdx.x;  // longest rows first when positions grow with t
  int n;
  const int32_t* pmap = nullptr;
  if (cm.pos) {
    // candidate list of a fused score + Top-K pass: every range but the last
    // contributes exactly cm.K entries (see index_topk.hip)
    const int nk = clampi(s.q_pos[t], -1, s.max_visible - 1) + 1;
    const int R = (nk + cm.range_keys - 1) / cm.range_keys;
    const int last = nk - (R - 1) * cm.range_keys;
    n = R ? (R - 1) * cm.K + (last < cm.K ? last : cm.K) : 0;
    pmap = cm.pos + (int64_t)t * ld;
  } else {
    const int64_t lim = ld < (int64_t)s.max_visible ? ld : (int64_t)s.max_visible;
    n = clampi(s.q_pos[t], -1, (int)lim - 1) + 1;
  }
  if (n <= n_lo || n > n_hi) return;
  const float* row = scores + (int64_t)t * ld;
  int32_t* orow = idx + (int64_t)t * K;
  float* vrow = vals ? vals + (int64_t)t * K : nullptr;

  const int sel = n < K ? n : K;
  for (int i = (sel > 0 ? sel : 0) + tid; i < K; i += kNT) {
    orow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
  if (sel <= 0) return;
  const int words = (n + 31) >> 5;
  if (order == 1 && words > FastSmem<PER>::kWords) {
    topk_exact(row, n, K, order, orow, vrow, pmap, smem.x);
    return;
  }

  for (int i = tid; i < kBins; i += kNT) {
    sh.hs[i] = 0;
    sh.hist[i] = 0;
    sh.cur[i] = 0;
  }
  if (order == 1)
    for (int i = tid; i < words; i += kNT) sh.bitmap[i] = 0;

  // ---- 1. keys, range, sample ----------------------------------------------------
  uint32_t key[PER > 0 ? PER : 1];
  if constexpr (PER > 0) {
    // Every load is unconditional, so that a batch is in flight together
    // instead of one branch, and one memory latency, per group of four.  The
    // row goes through a buffer descriptor whose range ends at the last whole
    // group of four holding a visible key (ld is a multiple of 4, so that
    // group is inside the row): loads of later groups return zeros without a
    // memory access, and each load needs only the lane's base offset plus a
    // scalar one.  Keys past n are masked to 0.
    const __amdgpu_buffer_rsrc_t rrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, ((n + 3) & ~3) * 4, kRawBuffer);
    const int ltid = opaque_tid();
    // eight loads in flight per thread at a time: all sixteen of the 64-key
    // form would not fit the registers of sixteen waves
    constexpr int kBatch = PER / 4 < kStreamLoads ? PER / 4 : kStreamLoads;
    static_assert((PER / 4) % kBatch == 0, "whole batches of loads");
#pragma unroll
    for (int j0 = 0; j0 < PER / 4; j0 += kBatch) {
      v4i v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rrs, ltid * 16, (j0 + u) * kNT * 16, 0));
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + u, i = (j * kNT + ltid) * 4;
        // all-ones for positions below n, from the sign of (position - n)
#pragma unroll
        for (int q = 0; q < 4; ++q) key[4 * j + q] = f2key(__int_as_float(v[u][q])) & (uint32_t)((i + q - n) >> 31);
      }
    }
  } else {
    key[0] = 0u;
  }
  // positions of this thread's candidates (same slots as the keys)
  int cpos[kCarry ? PER : 1];
  if constexpr (kCarry) {
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc((void*)pmap, 0, ((n + 3) & ~3) * 4, kRawBuffer);
    const int ltid = opaque_tid();
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(prs, ltid * 16, j * kNT * 16, 0));
#pragma unroll
      for (int q = 0; q < 4; ++q) cpos[4 * j + q] = v[q];
    }
  }
  uint32_t kmn = 0xffffffffu, kmx = 0u;
  for_keys<PER>(key, row, n, [&](uint32_t k, int, int) {
    kmn = min(kmn, k ? k : 0xffffffffu);
    kmx = max(kmx, k);
  });
  const bool sampled = n > kDirect;
  uint32_t smp = 0u;
  if (sampled) {
    if constexpr (PER > 0) {
      const int jn = min(PER / 4, (n + 4 * kNT - 1) / (4 * kNT));
      const int sidx = (tid % jn) * 4 + ((tid / jn) & 3);
#pragma unroll
      for (int i = 0; i < PER; ++i) smp = i == sidx ? key[i] : smp;
    } else {
      smp = f2key(row[(int)(((int64_t)tid * n) / kNT)]);
    }
  }
  kmn = wave_all(kmn, 0xffffffffu, OpMin{});
  kmx = wave_all(kmx, 0u, OpMax{});
  const uint32_t wns = (uint32_t)__popcll(__ballot(smp != 0u));
  if (lane == 0) {
    sh.red[0][w] = kmn;
    sh.red[1][w] = kmx;
    sh.red[2][w] = wns;
  }
  __syncthreads();
  const uint32_t kmin = waves_all<kNW>(sh.red[0], 0xffffffffu, OpMin{});
  const uint32_t kmax = waves_all<kNW>(sh.red[1], 0u, OpMax{});
  const uint32_t nsamp = waves_all<kNW>(sh.red[2], 0u, OpAdd{});
  if (kmax < kmin) {  // no finite score in the row
    topk_exact(row, n, K, order, orow, vrow, pmap, smem.x);
    return;
  }
  const int hb = kBins - 1 - 2 * tid;  // this thread's two bins, counted from the top

  // ---- lower bound L from the sample ------------------------------------------------
  uint32_t L = kmin;
  if (sampled && nsamp > 0) {
    const float e = (float)K * (float)nsamp / (float)n;  // expected samples above the K-th key
    uint32_t r = (uint32_t)ceilf(1.25f * e + 4.0f * sqrtf(e) + 4.0f);
    r = r < nsamp ? r : nsamp;
    const int shs = bin_shift((uint64_t)kmax - kmin + 1);
    if (smp) atomicAdd(&sh.hs[(smp - kmin) >> shs], 1u);
    __syncthreads();
    const uint32_t c0 = sh.hs[hb], c1 = sh.hs[hb - 1];
    uint32_t tot;
    const uint32_t a0 = block_excl<kNW>(c0 + c1, sh.scan[0], tot);
    const uint32_t a1 = a0 + c0;
    if (a0 < r && r <= a0 + c0) sh.L = kmin + ((uint32_t)hb << shs);
    if (a1 < r && r <= a1 + c1) sh.L = kmin + ((uint32_t)(hb - 1) << shs);
    __syncthreads();
    L = sh.L;
  }

  // ---- 2. histogram of the keys >= L ---------------------------------------------
  const int sh2 = bin_shift((uint64_t)kmax - L + 1);
  for_keys<PER>(key, row, n, [&](uint32_t k, int, int) {
    if (k >= L) atomicAdd(&sh.hist[(k - L) >> sh2], 1u);
  });
  __syncthreads();
  const uint32_t usel = (uint32_t)sel;
  uint32_t cand;
  {
    const uint32_t m0 = sh.hist[hb], m1 = sh.hist[hb - 1];
    const uint32_t a0 = block_excl<kNW>(m0 + m1, sh.scan[1], cand);
    const uint32_t a1 = a0 + m0;
    sh.above[hb] = a0;
    sh.above[hb - 1] = a1;
    if (a0 < usel && usel <= a0 + m0) {
      sh.bstar = (uint32_t)hb;
      sh.estar = a0 + m0;
    }
    if (a1 < usel && usel <= a1 + m1) {
      sh.bstar = (uint32_t)(hb - 1);
      sh.estar = a1 + m1;
    }
    uint32_t mm = max(a0 < usel ? m0 : 0u, a1 < usel ? m1 : 0u);
    mm = wave_all(mm, 0u, OpMax{});
    if (lane == 0) sh.maxm[w] = mm;
  }
  __syncthreads();
  if (cand < usel) {
    topk_exact(row, n, K, order, orow, vrow, pmap, smem.x);
    return;
  }
  const uint32_t bstar = sh.bstar, estar = sh.estar;
  const uint32_t maxm = waves_all<kNW>(sh.maxm, 0u, OpMax{});
  if (estar > (uint32_t)kBuf || maxm > (uint32_t)kMaxBin) {
    topk_exact(row, n, K, order, orow, vrow, pmap, smem.x);
    return;
  }

  // ---- 3. scatter bins >= b*, rank inside each bin ---------------------------------
  for_keys<PER>(key, row, n, [&](uint32_t k, int p, int slot) {
    if (k >= L) {
      const uint32_t b = (k - L) >> sh2;
      // carrying positions, the composite holds the key's position itself
      // (candidates are in position order, so the order of ties is unchanged)
      int tag = p;
      if constexpr (kCarry) tag = order == 0 ? cpos[slot < 0 ? 0 : slot] : p;
      if (b >= bstar) sh.buf[sh.above[b] + atomicAdd(&sh.cur[b], 1u)] = composite(k, tag);
    }
  });
  __syncthreads();
  for (int i = tid; i < (int)estar; i += kNT) {
    const uint64_t v = sh.buf[i];
    const uint32_t k = ~(uint32_t)(v >> 32);
    const uint32_t b = (k - L) >> sh2;
    const uint32_t st = sh.above[b], m = sh.hist[b];
    uint32_t rank = 0;
    for (uint32_t j = st; j < st + m; ++j) rank += sh.buf[j] < v;
    const uint32_t fin = st + rank;
    if (fin < usel) {
      const int p = (int)(uint32_t)v;
      if (order == 0) {
        orow[fin] = (pmap && !kCarry) ? pmap[p] : p;
        if (vrow) vrow[fin] = key2f(k);
      } else {
        atomicOr(&sh.bitmap[p >> 5], 1u << (p & 31));
      }
    }
  }
  if (order == 0) return;

  // order 1: compact the bitmap in position order
  __syncthreads();
  const int wpt = (words + kNT - 1) / kNT;
  const int w0 = tid * wpt;
  uint32_t c = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < words) c += __popc(sh.bitmap[w0 + i]);
  uint32_t tot;
  uint32_t off = block_excl<kNW>(c, sh.scan[2], tot);
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i >= words) break;
    uint32_t bits = sh.bitmap[w0 + i];
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      bits &= bits - 1;
      const int p = (w0 + i) * 32 + bpos;
      orow[off] = pmap ? pmap[p] : p;
      if (vrow) vrow[off] = key2f(f2key(row[p]));
      ++off;
    }
  }
}

template <int PER, bool CAND>
static hipError_t launch_rows_as(const float* scores, int64_t ld, const SeqArgs& s, int K, int order, int32_t* idx,
                                 float* vals, const CandMap& cm, int n_lo, int n_hi, hipStream_t st) {
  const size_t shm = sizeof(TopkSmem<PER>);
  hipError_t e =
      hipFuncSetAttribute((const void*)k_topk<PER, CAND>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_topk<PER, CAND>), dim3(s.T), dim3(kNT), shm, st, scores, ld, s, K, order, idx, vals, cm, n_lo,
                     n_hi);
  return hipGetLastError();
}
template <int PER>
static hipError_t launch_rows(const float* scores, int64_t ld, const SeqArgs& s, int K, int order, int32_t* idx,
                              float* vals, const CandMap& cm, hipStream_t st, int n_lo = -1,
                              int n_hi = 0x7fffffff) {
  return cm.pos ? launch_rows_as<PER, true>(scores, ld, s, K, order, idx, vals, cm, n_lo, n_hi, st)
                : launch_rows_as<PER, false>(scores, ld, s, K, order, idx, vals, cm, n_lo, n_hi, st);
}

// The rows of one call can differ in length (causal prefill: 1 .. max_visible
// keys).  With many rows, each row goes to the smallest variant that holds
// it, one launch per length class (the other classes' workgroups return at
// once): variants with fewer keys per thread use fewer registers and run more
// workgroups per CU, and rows that fit in registers are not streamed.  Few
// rows (decode) keep one launch.
constexpr int kClassMinRows = 1024;

hipError_t launch_topk(const float* scores, int64_t ld, const SeqArgs& s, int K, int order, int32_t* idx,
                       float* vals, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int64_t lim = ld < (int64_t)s.max_visible ? ld : (int64_t)s.max_visible;
  const CandMap none{nullptr, 0, 0};
  const bool split = s.T >= kClassMinRows;
  constexpr int c8 = kNT * 8, c32 = kNT * 32, c64 = kNT * 64;
  hipError_t e;
  if (lim <= c8) return launch_rows<8>(scores, ld, s, K, order, idx, vals, none, st);
  if (split && (e = launch_rows<8>(scores, ld, s, K, order, idx, vals, none, st, -1, c8)) != hipSuccess) return e;
  const int lo32 = split ? c8 : -1, lo64 = split ? c32 : -1, lo0 = split ? c64 : -1;
  if (lim <= c32) return launch_rows<32>(scores, ld, s, K, order, idx, vals, none, st, lo32);
  if (split && (e = launch_rows<32>(scores, ld, s, K, order, idx, vals, none, st, c8, c32)) != hipSuccess) return e;
  if (lim <= c64) return launch_rows<64>(scores, ld, s, K, order, idx, vals, none, st, lo64);
  if (split && (e = launch_rows<64>(scores, ld, s, K, order, idx, vals, none, st, c32, c64)) != hipSuccess) return e;
  return launch_rows<0>(scores, ld, s, K, order, idx, vals, none, st, lo0);
}

hipError_t launch_topk_candidates(const float* cscore, const int32_t* cpos, int64_t ldc, int range_keys,
                                  const SeqArgs& s, int K, int order, int32_t* idx, float* vals, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const CandMap cm{cpos, range_keys, K};
  if (ldc <= kNT * 8) return launch_rows<8>(cscore, ldc, s, K, order, idx, vals, cm, st);
  if (ldc <= kNT * 32) return launch_rows<32>(cscore, ldc, s, K, order, idx, vals, cm, st);
  if (ldc <= kNT * 64) return launch_rows<64>(cscore, ldc, s, K, order, idx, vals, cm, st);
  return launch_rows<0>(cscore, ldc, s, K, order, idx, vals, cm, st);
}

}  // namespace sia

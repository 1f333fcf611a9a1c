// Step 2 — per-query Top-K over the visible scores.
//
// [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models",
//      section "Sparse Attention Pipeline Optimization": keep the K best-scored
//      history positions of each query.
// [P2] "Efficient Inference Deployment and Optimization for Hybrid Attention
//      LLMs", section 3.2: Top-K consumes the index scores.
//
// Selected set: the first min(K, n) positions under (score desc, position asc),
// with -0 == +0.  One workgroup per query row.
//
//  1. Scores are mapped to order-preserving 32-bit keys (cached in LDS when the
//     row fits).  The row's key range [kmin, kmax] is found first.
//  2. Range-adaptive radix select: each pass histograms the keys inside the
//     current range into <= 2048 equal-width bins (LDS atomics, with a
//     wave-uniform fast path for runs of equal bins), walks the histogram from
//     the top to the bin holding the K-th key, and narrows the range to that
//     bin.  A 32-bit range closes in at most three passes.  The result is the
//     threshold key T and the number `need` of keys equal to T to keep.
//  3. One ordered pass (block-wide prefix sums built from wave ballots/scans)
//     keeps every key > T and the first `need` keys == T in position order,
//     which is the deterministic tie-break toward lower positions.
//  4. order 0 sorts the kept (key desc, position asc) pairs with a bitonic
//     network in LDS; order 1 writes them in ascending position directly.
#include "sia_common.hpp"
#include "sia_internal.hpp"

namespace sia {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kMaxK = 2048;
constexpr int kCacheKeys = 32768;

struct TopkShared {
  uint32_t hist[kBins];
  uint64_t sel[kMaxK];
  uint32_t red[2 * kTopkWaves];
  uint32_t scan[kTopkWaves];
  uint32_t found_bin;
  uint32_t found_above;
};

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int i = 1; i < kTopkWaves; ++i) r = min(r, red[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int i = 1; i < kTopkWaves; ++i) r = max(r, red[i]);
  __syncthreads();
  return r;
}

// Exclusive prefix sum over the block (thread order); returns the block total in *total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scan, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) scan[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t x = scan[i];
    before += (i < w) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

template <bool CACHED>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ scores, int64_t ld, SeqArgs s,
                                                       int K, int order, int32_t* __restrict__ idx,
                                                       float* __restrict__ vals) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  TopkShared& sh = *reinterpret_cast<TopkShared*>(smem_raw);
  uint32_t* cache = reinterpret_cast<uint32_t*>(smem_raw + sizeof(TopkShared));

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  int64_t lim = ld < (int64_t)s.max_visible ? ld : (int64_t)s.max_visible;
  const int pos = clampi(s.q_pos[t], -1, (int)lim - 1);
  const int n = pos + 1;
  const float* row = scores + (int64_t)t * ld;
  int32_t* orow = idx + (int64_t)t * K;
  float* vrow = vals ? vals + (int64_t)t * K : nullptr;

  auto key_at = [&](int i) -> uint32_t { return CACHED ? cache[i] : f2key(row[i]); };

  // ---- 1. keys and their range -------------------------------------------
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if (n > K) {
    const int n4 = n & ~3;
    for (int i = tid * 4; i < n4; i += kTopkThreads * 4) {
      const float4 f = *reinterpret_cast<const float4*>(row + i);
      const uint32_t k0 = f2key(f.x), k1 = f2key(f.y), k2 = f2key(f.z), k3 = f2key(f.w);
      if (CACHED) {
        cache[i] = k0; cache[i + 1] = k1; cache[i + 2] = k2; cache[i + 3] = k3;
      }
      kmin = min(min(kmin, min(k0, k1)), min(k2, k3));
      kmax = max(max(kmax, max(k0, k1)), max(k2, k3));
    }
    for (int i = n4 + tid; i < n; i += kTopkThreads) {
      const uint32_t k0 = f2key(row[i]);
      if (CACHED) cache[i] = k0;
      kmin = min(kmin, k0);
      kmax = max(kmax, k0);
    }
    kmin = block_min_u32(kmin, sh.red);
    kmax = block_max_u32(kmax, sh.red + kTopkWaves);
  } else if (CACHED) {
    for (int i = tid; i < n; i += kTopkThreads) cache[i] = f2key(row[i]);
    __syncthreads();
  }

  // ---- 2. threshold key ----------------------------------------------------
  uint32_t T = 0u;
  uint32_t need = 0u;
  if (n > K) {
    uint32_t lo = kmin;
    uint64_t range = (uint64_t)kmax - kmin + 1;
    need = (uint32_t)K;
    while (range > 1) {
      const int bits = 64 - __clzll((long long)(range - 1));
      const int shift = bits > 11 ? bits - 11 : 0;
      const int nb = (int)((range - 1) >> shift) + 1;
      for (int i = tid; i < nb; i += kTopkThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t k = key_at(i);
        const bool in = (uint64_t)(k - lo) < range && k >= lo;
        const uint32_t bin = (k - lo) >> shift;
        const uint64_t m = __ballot(in);
        if (m) {
          const int first = __ffsll((unsigned long long)m) - 1;
          const uint32_t fb = (uint32_t)__shfl((int)bin, first, 64);
          const uint64_t same = __ballot(in && bin == fb);
          if (same == m) {
            if (lane == first) atomicAdd(&sh.hist[fb], (uint32_t)__popcll(m));
          } else if (in) {
            atomicAdd(&sh.hist[bin], 1u);
          }
        }
      }
      __syncthreads();
      // thread i owns bins [4i, 4i+4); suffix sums from the top bin down
      const int b0 = tid * 4;
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) c += (b0 + j < nb) ? sh.hist[b0 + j] : 0u;
      // suffix (exclusive) over threads: count in bins above my range
      uint32_t tot;
      const uint32_t pre = block_excl_scan(c, sh.scan, &tot);
      const uint32_t above = tot - pre - c;
      if (above < need && need <= above + c) {
        uint32_t acc = above;
        for (int j = 3; j >= 0; --j) {
          const int bj = b0 + j;
          if (bj >= nb) continue;
          const uint32_t hj = sh.hist[bj];
          if (acc + hj >= need) {
            sh.found_bin = (uint32_t)bj;
            sh.found_above = acc;
            break;
          }
          acc += hj;
        }
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

  // ---- 3. ordered selection ------------------------------------------------
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += kTopkThreads * 4) {
    uint32_t kk[4];
    int cnt_gt = 0, cnt_eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + tid * 4 + j;
      kk[j] = i < n ? key_at(i) : 0u;
      cnt_gt += kk[j] > T;
      cnt_eq += (i < n) && kk[j] == T && need > 0;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan((uint32_t)cnt_gt | ((uint32_t)cnt_eq << 16), sh.scan, &tot);
    uint32_t g = run_gt + (pre & 0xffffu), e = run_eq + (pre >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + tid * 4 + j;
      const bool gt = kk[j] > T;
      const bool eq = (i < n) && kk[j] == T && need > 0;
      if (gt || (eq && e < need)) {
        const uint32_t slot = g + (e < need ? e : need);
        sh.sel[slot] = ((uint64_t)(~kk[j]) << 32) | (uint32_t)i;
      }
      g += gt;
      e += eq;
    }
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
  __syncthreads();

  // ---- 4. output -------------------------------------------------------------
  const int cnt = n < K ? (n > 0 ? n : 0) : K;
  if (order == 0 && cnt > 1) {
    int P = 1;
    while (P < cnt) P <<= 1;
    for (int i = cnt + tid; i < P; i += kTopkThreads) sh.sel[i] = ~0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P / 2; i += kTopkThreads) {
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
  for (int i = tid; i < K; i += kTopkThreads) {
    if (i < cnt) {
      const uint64_t v = sh.sel[i];
      orow[i] = (int32_t)(uint32_t)v;
      if (vrow) vrow[i] = key2f(~(uint32_t)(v >> 32));
    } else {
      orow[i] = -1;
      if (vrow) vrow[i] = -INFINITY;
    }
  }
}

hipError_t launch_topk(const float* scores, int64_t ld, const SeqArgs& s, int K, int order, int32_t* idx,
                       float* vals, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int64_t lim = ld < (int64_t)s.max_visible ? ld : (int64_t)s.max_visible;
  if (lim <= kCacheKeys) {
    const size_t shm = sizeof(TopkShared) + (size_t)kCacheKeys * 4;
    hipError_t e = hipFuncSetAttribute((const void*)k_topk<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_topk<true>, dim3(s.T), dim3(kTopkThreads), shm, st, scores, ld, s, K, order, idx, vals);
  } else {
    hipLaunchKernelGGL(k_topk<false>, dim3(s.T), dim3(kTopkThreads), sizeof(TopkShared), st, scores, ld, s, K,
                       order, idx, vals);
  }
  return hipGetLastError();
}

}  // namespace sia

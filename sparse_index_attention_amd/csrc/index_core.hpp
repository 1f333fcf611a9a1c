// Indexer scoring shared by the score kernel and the fused score + Top-K kernel.
//
//   score[t, s] = sum_h w[t,h] * ReLU(qs[t,h] * ks[s] * <q[t,h], k[s]>),  s <= q_pos[t]
//
// [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models",
//      section "Sparse Attention Pipeline Optimization"; [P2] "Efficient
//      Inference Deployment and Optimization for Hybrid Attention LLMs", section 3.1.
#pragma once
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

__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One wave scores query t against the 64-key pages [c_begin, c_end) of its
// sequence's block table and calls sink(s, score) once per page with lane l
// holding key s = 64c + l (scores of keys past pos are -inf).
// Lane l: nn = l % 32 (key within an N tile / head within an M tile), hh = l / 32.
// K-step mapping (same for both operands): step st of lane half hh covers
// depth bytes [64*hh + 32*st, 64*hh + 32*st + 32).
template <int HI, typename Sink>
__device__ __forceinline__ void score_pages(const IndexArgs& a, int t, int pos, int b, int c_begin, int c_end,
                                            Sink&& sink) {
  constexpr int MT = HI / 32;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, nn = lane & 31;
  const uint8_t* __restrict__ kpool = (const uint8_t*)a.k_pool;
  const uint8_t* __restrict__ qbase = (const uint8_t*)a.q;
  const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;

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
        // ReLU as an integer max: negative floats (and -0) have the sign bit
        // set, so max(bits, 0) is 0 for them and the identity otherwise (one
        // instruction; fmaxf would also quiet NaNs first)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum = fmaf(wr[mt][r], __int_as_float(max(__float_as_int(acc[r]), 0)), sum);
      }
      p[kt] = sum;
    }
    // lane l < 32 holds half of the heads of keys l (p[0]) and 32+l (p[1]),
    // lane 32+l the other half: swap the cross halves, then one add gives lane
    // l the score of key 64*c + l
    const auto hv = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
    float score = (__uint_as_float(hv[0]) + __uint_as_float(hv[1])) * ks;
    const int s = c * 64 + lane;
    if (s > pos) score = -INFINITY;
    sink(s, score);
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

}  // namespace sia

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

// s_waitcnt immediate (gfx9 encoding): vmcnt(0), no wait on expcnt or lgkmcnt
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

struct IndexArgs {
  const void* q;
  const float* q_scale;   // fp8: per token or per (token, head)
  const float* w;
  const void* k_pool;
  const float* k_scale;   // fp8: per key token
  const uint8_t* q_mx;    // MXFP8: [T, H, 4] E8M0 group scales (groups of 32 along dim)
  const uint8_t* k_mx;    // MXFP8: [pages, 64, 4]
  int q_scale_per_head;
  int H;
  int D;
  SeqArgs s;
  float* scores;
  int64_t ld;
};

inline IndexArgs index_args(const sia_indexer_in& in, const SeqArgs& s, float* scores, int64_t ld) {
  const bool mx = in.dtype == SIA_MXFP8_E4M3;
  return IndexArgs{in.q, mx ? nullptr : (const float*)in.q_scale, in.w, in.k_pool,
                   mx ? nullptr : (const float*)in.k_scale, mx ? (const uint8_t*)in.q_scale : nullptr,
                   mx ? (const uint8_t*)in.k_scale : nullptr, in.q_scale_per_head, in.heads, in.dim, s, scores, ld};
}

// Zero scale operands select the unscaled instruction (unit scales).
__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Block-scaled form for MXFP8.  In this instruction the 32 bytes of a lane
// of row (or column) m split into two K blocks of the MFMA: bytes 0..15 of
// lanes m and m+32 form block 0, bytes 16..31 of both form block 1, and the
// scale of block b comes from lane m + 32b (byte ST of its scale register for
// K step ST).  The MX operands are therefore laid out so that a block is one
// 32-element group: K step st, lane half hh holds depth [64st + 16hh, +16)
// in bytes 0..15 and [64st + 32 + 16hh, +16) in bytes 16..31 (groups 2st and
// 2st + 1), and lane half hh supplies the scale of group 2st + hh.
template <int ST>
__device__ __forceinline__ v16f mfma_mx(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, ST, (int)sa, ST, (int)sb);
}

// The scale bytes a lane supplies, from its row's four group scales (bytes
// g0..g3 of row_word): byte st = group 2st + hh.
__device__ __forceinline__ uint32_t mx_lane_scales(uint32_t row_word, int hh) {
  const uint32_t w = hh ? row_word >> 8 : row_word;
  return (w & 0xffu) | ((w >> 8) & 0xff00u);
}

// MX operand of K step ST from a 128-byte row: depth [64ST + 16hh, +16) and
// [64ST + 32 + 16hh, +16).
template <int ST>
__device__ __forceinline__ v8i mx_operand(const uint8_t* row, int hh) {
  const v4i lo = *(const v4i*)(row + 64 * ST + 16 * hh);
  const v4i hi = *(const v4i*)(row + 64 * ST + 32 + 16 * hh);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One wave scores query t against 64-key pages of its sequence and calls
// sink(s, score) once per page with lane l holding key s = 64c + l (scores of
// keys past pos are -inf).  The pages are c = claim(), claim(), ... until
// claim() returns -1; claim() must return a wave-uniform value and, once it
// has returned -1, keep doing so.  page_of(c) gives the physical page of
// logical page c (wave-uniform).  It must not read global memory: a vector
// memory load in the loop would make the wave wait for every page load in
// flight before it (their counter drains in order), which empties the ring.
// Lane l: nn = l % 32 (key within an N tile / head within an M tile), hh = l / 32.
// K-step mapping (same for both operands): step st of lane half hh covers
// depth bytes [64*hh + 32*st, 64*hh + 32*st + 32).
// MX: MXFP8 inputs (group scales inside the MFMA; no per-token scales).
template <int HI, bool MX, typename Claim, typename PageOf, typename Sink>
__device__ __forceinline__ void score_claimed_pages(const IndexArgs& a, int t, int pos, Claim&& claim,
                                                    PageOf&& page_of, Sink&& sink) {
  constexpr int MT = HI / 32;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, nn = lane & 31;
  const uint8_t* __restrict__ kpool = (const uint8_t*)a.k_pool;
  const uint8_t* __restrict__ qbase = (const uint8_t*)a.q;

  // key pages go through a ring of three register buffers: while page c is
  // computed, pages c+1 and c+2 are in flight
  // ks: fp8 key scale of key 64c + lane; MX: the group-scale words of keys
  // nn (kt = 0) and 32 + nn (kt = 1) of the page, as this lane uses them
  struct KScale {
    float f;
    uint32_t w[2];
  };
  // Every page request is unconditional: the page goes through a buffer
  // descriptor built in scalar registers, and for c < 0 (nothing left to
  // claim) the descriptor's range is empty, so the loads return zeros without
  // a memory access.  With conditional requests the compiler could not count
  // the loads in flight and waited for all of them before each page's first
  // MFMAs, which kept about one page in flight per wave instead of two.
  auto load_page = [&](int c, v8i (&kb)[2][2], KScale& ks) __attribute__((always_inline)) {
    c = __builtin_amdgcn_readfirstlane(c);   // wave-uniform: the descriptors stay in scalar registers
    int page = page_of(c);
    page = page < 0 ? 0 : (page >= a.s.num_pages ? a.s.num_pages - 1 : page);
    page = __builtin_amdgcn_readfirstlane(page);
    const bool ok = c >= 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kpool + (int64_t)page * (kPage * 128)), 0, ok ? kPage * 128 : 0, kRawBuffer);
    auto ld16 = [&](int off) __attribute__((always_inline)) {
      return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
    };
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int row = (32 * kt + nn) * 128;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        // MX: depth [64x + 16hh, +16) and [64x + 32 + 16hh, +16) (see mx_operand);
        // fp8: depth [64hh + 32x, +32)
        const int o0 = MX ? row + 64 * x + 16 * hh : row + 64 * hh + 32 * x;
        const int o1 = MX ? o0 + 32 : o0 + 16;
        const v4i lo = ld16(o0), hi = ld16(o1);
        kb[kt][x] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    const void* sbase = MX ? (const void*)(a.k_mx + (int64_t)page * kPage * 4) : (const void*)(a.k_scale + (int64_t)page * kPage);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, 0, ok ? kPage * 4 : 0, kRawBuffer);
    if constexpr (MX) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        ks.w[kt] = mx_lane_scales(__builtin_amdgcn_raw_buffer_load_b32(srs, (32 * kt + nn) * 4, 0, 0), hh);
    } else {
      ks.f = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4, 0, 0));
    }
    // keep the requests here: without this the compiler sinks them past the
    // loop's exit test into the next step, one page later
    asm volatile("" ::: "memory");
  };
  v8i k0[2][2], k1[2][2], k2[2][2];
  KScale ks0{}, ks1{}, ks2{};
  int c0 = claim();
  if (c0 < 0) return;
  load_page(c0, k0, ks0);
  int c1 = claim();
  load_page(c1, k1, ks1);
  int c2 = claim();
  load_page(c2, k2, ks2);

  // query operand (A): head m = 32*mt + nn
  v8i qa[MT][2];
  uint32_t qsc[MT];   // MX: group scales of head 32mt + nn
  float wr[MT][16];
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
  // Everything loaded so far (the first three pages, the query and its
  // weights) lands before the loop starts.  Otherwise the compiler's wait for
  // the query operand, needed on the first pass only, stays at the loop head
  // as a wait for every load in flight and runs on every pass.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  // scores of page c from buffer kb, then buffer kb takes the next claimed
  // page (returned; -1 when none is left)
  auto step = [&](int c, v8i (&kb)[2][2], KScale& ks) __attribute__((always_inline)) -> int {
    if (c >= 0) {   // wave-uniform; the buffer's request below is unconditional
    float p[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v16f acc = {};
        if constexpr (MX) {
          acc = mfma_mx<0>(qa[mt][0], kb[kt][0], acc, qsc[mt], ks.w[kt]);
          acc = mfma_mx<1>(qa[mt][1], kb[kt][1], acc, qsc[mt], ks.w[kt]);
        } else {
          acc = mfma_f8(qa[mt][0], kb[kt][0], acc);
          acc = mfma_f8(qa[mt][1], kb[kt][1], acc);
        }
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
    float score = __uint_as_float(hv[0]) + __uint_as_float(hv[1]);
    if constexpr (!MX) score *= ks.f;
    const int s = c * 64 + lane;
    if (s > pos) score = -INFINITY;
    sink(s, score);
    }
    const int next = claim();
    load_page(next, kb, ks);
    return next;
  };
  // Pages are claimed in processing order, so once a round has claimed -1
  // for buffer 0 the two later buffers hold -1 as well.  The one exit test
  // per round keeps every path into the loop head the same: with an exit
  // after each step the compiler merged the exits into a path that skipped
  // two buffers' requests, and waited for every load in flight at the head.
  while (true) {
    c0 = step(c0, k0, ks0);
    c1 = step(c1, k1, ks1);
    c2 = step(c2, k2, ks2);
    if (c0 < 0) break;
  }
}

// The pages [c_begin, c_end) in order, c_begin < c_end <= c_begin + 64.
// Their physical pages are loaded once, one per lane (lane l: page
// c_begin + l), and read with a lane select.
template <int HI, bool MX, typename Sink>
__device__ __forceinline__ void score_pages(const IndexArgs& a, int t, int pos, int b, int c_begin, int c_end,
                                            Sink&& sink) {
  const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;
  const int lane = threadIdx.x & 63;
  const int win = table[min(c_begin + lane, c_end - 1)];
  int next = c_begin;
  score_claimed_pages<HI, MX>(
      a, t, pos, [&]() __attribute__((always_inline)) { return next < c_end ? next++ : -1; },
      [&](int c) __attribute__((always_inline)) {
        return __builtin_amdgcn_readlane(win, __builtin_amdgcn_readfirstlane(max(c - c_begin, 0)));
      },
      sink);
}

}  // namespace sia

// Wave- and block-level primitives shared by the Top-K kernels (gfx950, wave64).
#pragma once
#include "sia_common.hpp"

namespace sia {

struct OpAdd {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct OpMin {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct OpMax {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp(uint32_t id, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWMASK, 0xf, false);
}
// Inclusive scan inside each row of 16 lanes (row_shr 1, 2, 4, 8).
template <typename Op>
__device__ __forceinline__ uint32_t row_incl(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp<0x111, 0xf>(id, v));
  v = op(v, dpp<0x112, 0xf>(id, v));
  v = op(v, dpp<0x114, 0xf>(id, v));
  v = op(v, dpp<0x118, 0xf>(id, v));
  return v;
}
// Inclusive scan over the wave in lane order (rows joined with row_bcast 15/31).
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl(uint32_t v, uint32_t id, Op op) {
  v = row_incl(v, id, op);
  v = op(v, dpp<0x142, 0xa>(id, v));
  v = op(v, dpp<0x143, 0xc>(id, v));
  return v;
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_all(uint32_t v, uint32_t id, Op op) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl(v, id, op), 63);
}
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Combines one value per wave (slot[NW], NW <= 16, written before the last barrier).
template <int NW, typename Op>
__device__ __forceinline__ uint32_t waves_all(const uint32_t* slot, uint32_t id, Op op) {
  const int lane = threadIdx.x & 63;
  const uint32_t x = lane < NW ? slot[lane] : id;
  return (uint32_t)__builtin_amdgcn_readlane((int)row_incl(x, id, op), NW - 1);
}

// Exclusive prefix sum over a block of NW waves in thread order, and the block
// total.  One barrier inside; `slot` (NW words) must not be written again before
// the next barrier that every thread passes after this call.
template <int NW>
__device__ __forceinline__ uint32_t block_excl(uint32_t v, uint32_t* slot, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = wave_index();
  const uint32_t inc = wave_incl(v, 0u, OpAdd{});
  if (lane == 63) slot[w] = inc;
  __syncthreads();
  const uint32_t x = row_incl(lane < NW ? slot[lane] : 0u, 0u, OpAdd{});
  const uint32_t before = w ? (uint32_t)__builtin_amdgcn_readlane((int)x, w - 1) : 0u;
  total = (uint32_t)__builtin_amdgcn_readlane((int)x, NW - 1);
  return before + inc - v;
}

// Shift that maps a key range of `range` values onto at most 2048 bins.
__device__ __forceinline__ int bin_shift(uint64_t range) {
  const int bits = range > 1 ? 64 - __clzll((long long)(range - 1)) : 0;
  return bits > 11 ? bits - 11 : 0;
}

// (key desc, position asc) is the ascending order of this composite.
__device__ __forceinline__ uint64_t composite(uint32_t key, int pos) {
  return ((uint64_t)(~key) << 32) | (uint32_t)pos;
}

}  // namespace sia

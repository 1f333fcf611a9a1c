// Device-side helpers shared by the libsia kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sia {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int v8i;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int v4i;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float v4f;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float v16f;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 v8bf;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
constexpr int kPage = 64;
// buffer descriptor word 3: raw 32-bit data, range-checked (loads past the
// range return zeros without touching memory, stores past it are dropped)
constexpr int kRawBuffer = 0x00020000;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// bfloat16 bits <-> float
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float -> bfloat16 bits with the hardware round-to-nearest-even conversion.
__device__ __forceinline__ uint16_t f32_to_bf16_hw(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// 2^x on the transcendental unit (results below 2^-126 flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two packed e4m3 codes (byte 0/1 or 2/3 of `w`) -> two floats (exact).
template <bool HI>
__device__ __forceinline__ float2 fp8x2_to_f32(uint32_t w) {
  auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return make_float2(r[0], r[1]);
}

// Order-preserving map float -> uint32 (larger float => larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Wave-wide sums / max via cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Physical slot of logical position `pos` of a sequence, with the page id clamped
// into the pool so that no access leaves it.
__device__ __forceinline__ int64_t page_slot(const int32_t* __restrict__ table_row, int pos, int num_pages) {
  int page = table_row[pos >> 6];
  page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
  return (int64_t)page * kPage + (pos & (kPage - 1));
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace sia

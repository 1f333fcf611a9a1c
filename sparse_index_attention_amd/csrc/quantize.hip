// Dynamic quantization of the indexer's bf16 queries, the weight-free step of
// the indexer prolog.
//
// [P2] "Efficient Inference Deployment and Optimization for Hybrid Attention
//      LLMs", section 3.2: Q quantization runs in the prolog, on the decode
//      critical path.
// [P2] section 4.1, [P5] section 4 table: index Q/K in MXFP8, one shared
//      power-of-two scale per 32 elements.
//
// Per-token fp8: scale = amax / 448 over the token's heads x dim values and
// codes = e4m3(x * (448 / amax)), both divisions correctly rounded in fp32; a
// token of zeros gets scale 1 and zero codes.  MXFP8: per group of 32
// consecutive elements of a head's dim axis, the smallest 2^e with
// amax <= 448 * 2^e (E8M0 byte e + 127; 0 for an all-zero group) and codes =
// e4m3(x * 2^-e), an exact scaling.
#include "block_prims.hpp"
#include "sia_internal.hpp"

namespace sia {

// float -> OCP e4m3 code: nearest grid value with ties to the even code,
// saturating at 448, sign kept (-0 -> 0x80).  Finite inputs.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal codes, spacing 2^-9
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t au = __float_as_uint(a);
    uint32_t e4 = (au >> 23) - 127 + 7;        // 1 .. 15
    uint32_t m3 = (au >> 20) & 7u;             // top three mantissa bits
    const uint32_t rem = au & 0xfffffu, half = 0x80000u;
    if (rem > half || (rem == half && (m3 & 1u))) ++m3;
    if (m3 == 8u) {
      m3 = 0u;
      ++e4;
    }
    code = (e4 << 3) | m3;
    code = code > 0x7eu ? 0x7eu : code;
  }
  return code | sign;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// one workgroup per token; thread i converts elements [PER*i, PER*i + PER)
template <int PER>
__global__ __launch_bounds__(256) void k_quantize_q_fp8(const uint16_t* __restrict__ q, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scale, int per_token) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint4* src = (const uint4*)(q + (int64_t)t * per_token + PER * tid);
  uint4 w[PER / 8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER / 8; ++i) {
    w[i] = src[i];
    const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(u[j])), fabsf(bf16_hi(u[j]))));
  }
  // non-negative floats order like their bit patterns
  uint32_t am = wave_all(__float_as_uint(amax), 0u, OpMax{});
  if ((tid & 63) == 0) red[tid >> 6] = __uint_as_float(am);
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float r = amax > 0.f ? 448.f / amax : 0.f;
  if (tid == 0) scale[t] = amax > 0.f ? amax / 448.f : 1.f;
  uint32_t out[PER / 4];
#pragma unroll
  for (int i = 0; i < PER / 8; ++i) {
    const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t c0 = f32_to_e4m3(bf16_lo(u[2 * j]) * r), c1 = f32_to_e4m3(bf16_hi(u[2 * j]) * r);
      const uint32_t c2 = f32_to_e4m3(bf16_lo(u[2 * j + 1]) * r), c3 = f32_to_e4m3(bf16_hi(u[2 * j + 1]) * r);
      out[2 * i + j] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
  uint4* dst = (uint4*)(codes + (int64_t)t * per_token + PER * tid);
#pragma unroll
  for (int i = 0; i < PER / 16; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

// one thread per group of 32 elements
__global__ __launch_bounds__(256) void k_quantize_q_mx(const uint16_t* __restrict__ q, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t groups) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups) return;
  const uint4* src = (const uint4*)(q + g * 32);
  uint4 w[4];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = src[i];
    const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(u[j])), fabsf(bf16_hi(u[j]))));
  }
  int e = -127;
  if (amax > 0.f) {
    int E;
    const float m = frexpf(amax, &E);  // amax = m * 2^E, m in [0.5, 1)
    e = m <= 0.875f ? E - 9 : E - 8;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  scales[g] = (uint8_t)(e + 127);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t c0 = f32_to_e4m3(ldexpf(bf16_lo(u[2 * j]), -e)), c1 = f32_to_e4m3(ldexpf(bf16_hi(u[2 * j]), -e));
      const uint32_t c2 = f32_to_e4m3(ldexpf(bf16_lo(u[2 * j + 1]), -e));
      const uint32_t c3 = f32_to_e4m3(ldexpf(bf16_hi(u[2 * j + 1]), -e));
      out[2 * i + j] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
  uint4* dst = (uint4*)(codes + g * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

hipError_t launch_quantize_q(const void* q_bf16, int T, int heads, int dim, bool mx, uint8_t* codes, void* scales,
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int per_token = heads * dim;
  if (mx) {
    const int64_t groups = (int64_t)T * per_token / 32;
    hipLaunchKernelGGL(k_quantize_q_mx, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st,
                       (const uint16_t*)q_bf16, codes, (uint8_t*)scales, groups);
  } else if (per_token == 64 * 128) {
    hipLaunchKernelGGL(k_quantize_q_fp8<32>, dim3(T), dim3(256), 0, st, (const uint16_t*)q_bf16, codes,
                       (float*)scales, per_token);
  } else {
    hipLaunchKernelGGL(k_quantize_q_fp8<16>, dim3(T), dim3(256), 0, st, (const uint16_t*)q_bf16, codes,
                       (float*)scales, per_token);
  }
  return hipGetLastError();
}

}  // namespace sia

// Step 3 — sparse MLA attention over the Top-K rows of a paged latent cache.
//
// [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models",
//      section "Sparse Attention Pipeline Optimization": the sparse kernel reads
//      only the selected KV entries and runs block-wise fused attention on them.
// [P3] "Day-One Inference Adaptation for Very Large Hybrid-Attention Models",
//      section 3.2: tile by query block, aggregate over the selected positions,
//      stage tiles in on-chip shared memory.
// [P5] "Inference Adaptation and Performance Optimization for a Domestically
//      Developed LLM's New Architecture", section 4 table: FP8 KV cache with
//      per-token 128-element tiles (the per-page tile is also supported).
//
// MFMA path (bf16 / fp8 cache, latent 512 + rope 64): one workgroup = one query
// token (all heads) x a contiguous share of its selected rows.  Wave w owns heads
// [32w, 32w+32).  Per 32-row tile:
//   * rows are gathered from the paged cache straight into LDS (16-byte direct
//     global->LDS loads for bf16; fp8 rows go through registers and are
//     dequantized to bf16 on the way), double buffered;
//   * S^T[row, head] = KV_tile . Q^T on v_mfma_f32_32x32x16_bf16: the KV tile is
//     the LDS operand, the wave's 32 query heads stay in registers for the
//     whole token;
//   * softmax per head is lane-local (each lane owns one head column) against a
//     fixed per-head reference, so the accumulator is never rescaled;
//   * O^T[vcol, head] += V^T . P^T: P^T comes straight from the S^T accumulator
//     (the row order inside the MFMA K dimension is chosen to match it) and V^T
//     is read with ds_read_b64_tr_b16 transposing loads.
// The LDS tile is row-major (72 16-byte chunks per row) with the chunk index
// XOR-swizzled by a 3-bit function of row bits 1..3 (see swz), which keeps both
// the 128-bit row reads and the transposing reads free of bank conflicts on
// gfx950's 64 four-byte LDS banks.
//
// Decode splits a token's rows over several workgroups; each writes a partial
// (O normalised over its rows, rounded to bf16, and its LSE in float) and a
// combine kernel merges them with softmax weights exp(lse_s - LSE) in a fixed
// order.  The merge is a convex combination, so the bf16 partials add at most
// one more rounding of 2^-9 relative to the output's own.
#include "sia_common.hpp"
#include "sia_internal.hpp"

namespace sia {

struct MlaArgs {
  const void* q;
  const void* kv;
  const float* kv_scale;
  int scale_tokens, scale_elems;  // fp8 tiles (powers of two)
  int log2_scale_tokens, log2_scale_elems;
  int H;
  int Dc, Dr;
  SeqArgs s;
  const int32_t* idx;
  int K;
  float scale_log2;  // softmax_scale * log2(e)
  int splits;
  int rows_per_split;
  void* out;    // final output (splits == 1)
  float* lse;   // nullable
  uint16_t* ws_o;  // [T, splits, H, Dc] bf16 partial outputs (splits > 1)
  float* ws_lse;    // [T, splits, H]
};

// ---------------------------------------------------------------------------
// float32 path (small dims): one workgroup per (token, head).
// ---------------------------------------------------------------------------
constexpr int kF32MaxDim = 1024;
constexpr int kF32MaxK = 2048;

__global__ __launch_bounds__(256) void k_sparse_mla_f32(MlaArgs a) {
  __shared__ float sq[kF32MaxDim];
  __shared__ float sl[kF32MaxK];
  __shared__ int64_t sslot[kF32MaxK];
  __shared__ float red[8];
  const int t = blockIdx.x, h = blockIdx.y;
  const int D = a.Dc + a.Dr, tid = threadIdx.x;
  const int b = clampi(a.s.q_seq[t], 0, a.s.batch - 1);
  const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;
  const float* q = (const float*)a.q + ((int64_t)t * a.H + h) * D;
  const float* kv = (const float*)a.kv;
  for (int i = tid; i < D; i += blockDim.x) sq[i] = q[i];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < a.K; j += blockDim.x) {
    const int p = a.idx[(int64_t)t * a.K + j];
    float l = -INFINITY;
    int64_t slot = -1;
    if (p >= 0 && p < a.s.max_visible) {
      slot = page_slot(table, p, a.s.num_pages);
      const float* r = kv + slot * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[d], r[d], dot);
      l = dot * a.scale_log2;
    }
    sl[j] = l;
    sslot[j] = slot;
    mx = fmaxf(mx, l);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) mx = fmaxf(mx, red[i]);
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < a.K; j += blockDim.x) {
    const float p = sslot[j] >= 0 ? exp2f(sl[j] - mx) : 0.f;
    sl[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  sum = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) sum += red[i];
  float* out = (float*)a.out + ((int64_t)t * a.H + h) * a.Dc;
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int d = tid; d < a.Dc; d += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < a.K; ++j)
      if (sslot[j] >= 0) acc = fmaf(sl[j], kv[sslot[j] * D + d], acc);
    out[d] = acc * inv;
  }
  if (tid == 0 && a.lse)
    a.lse[(int64_t)t * a.H + h] = sum > 0.f ? (mx + log2f(sum)) * 0.6931471805599453f : -INFINITY;
}

// ---------------------------------------------------------------------------
// MFMA path.
// ---------------------------------------------------------------------------
constexpr int kDc = 512, kDr = 64, kD = kDc + kDr;
constexpr int kChunks = kD / 8;                   // 72 chunks of 8 bf16 (16 bytes) per row
constexpr int kRowsTile = 32;
// read for latent rows without a valid index when the pool is addressed directly
__device__ uint4 g_zero_kv_row[kD * 2 / 16];
constexpr int kTileBytes = kRowsTile * kD * 2;   // 36864

// Chunk swizzle of a tile row: bit 1 of the row -> bit 2, bit 3 -> bit 1, bit 2
// -> bit 0.  A 128-bit read of one chunk per row by 16 consecutive lanes (rows
// r..r+15) then covers all 64 banks once: even rows and odd rows each take all
// eight swizzle values.  A transposing read covers rows r..r+3 (r % 4 == 0),
// where rows two apart differ in swizzle bit 2 and so land in disjoint banks.
// Rows 16 apart share the swizzle.
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) & 1) << 2) | (((row >> 3) & 1) << 1) | ((row >> 2) & 1);
}

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) v4bf lds_v4bf;
typedef __attribute__((address_space(3))) v8bf lds_v8bf;
typedef __attribute__((address_space(3))) v4i lds_v4i;

__device__ __forceinline__ v4bf lds_tr16(lds_u8* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(base + byte_off));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_hw(lo) | ((uint32_t)f32_to_bf16_hw(hi) << 16);
}

// LDS tile layout: 72 chunks of 16 bytes per row, grouped 8 chunks at a time:
//   slot(row, c) = (c / 8) * 256 + row * 8 + ((c % 8) ^ swz(row)),  byte = 16 * slot.
// A wave's 16-byte direct load then fills 64 consecutive slots (8 rows x one
// 128-byte chunk group), and every LDS read is one per-lane base register plus a
// compile-time immediate.
//
// Work split.  A workgroup takes up to 64 heads of one (token, split): wave
// (hb, ch) owns head block hb (32 heads) and output column half ch (256 of the
// 512 latent columns), so its output accumulator is 128 registers.  The two
// waves of a head block split the score contraction instead of repeating it:
// wave ch multiplies depth steps 4g + 2ch and 4g + 2ch + 1 (g = 0..8) of the 36
// 16-deep steps, both write their partial S^T to LDS, and each adds the
// other's.  Each wave therefore keeps only its half of the query operand in
// registers (18 steps), and a tile costs a wave 18 + 16 MFMAs.  With 128 heads a
// (token, split) takes two workgroups.  All workgroups of a token run on one
// XCD (see the block mapping), so the second gather of a row and the splits'
// query loads are served by its L2.
constexpr int kVH = 256;
constexpr int kMaxSplitRows = 2048;      // rows of one split, slots resolved once per workgroup
constexpr int kHalfSteps = 18;           // score steps per wave
constexpr int kVT = kVH / 32;  // 32-column output tiles per half

// s_waitcnt immediate (gfx9 encoding): vmcnt = n (bits 3:0 and 15:14),
// expcnt = 7 (no wait), lgkmcnt = 0
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() { __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(N)); }

// RS (fp8 only): the latent part of a row has one scale (tiles of 512
// elements).  The codes are then staged exactly (e4m3 -> bf16 is exact), and
// the scale moves onto the row's latent score (s * S_latent + S_rope) and onto
// its softmax weight in P before the P.V product, instead of scaling each of
// the 512 elements while staging.
template <int NW, bool FP8, bool BUF, bool RS = false>
__global__ __launch_bounds__(NW * 64, 1) void k_sparse_mla_mfma(MlaArgs a) {
  constexpr int NT = NW * 64;
  constexpr int HBW = NW / 2;                  // head blocks per workgroup
  constexpr int TPR = NT / kRowsTile;          // threads per row in the fp8 gather
  constexpr int kFp8Loads = 40 / TPR;          // 640-byte rows = 40 loads of 16 bytes
  // three distinct LDS objects (not one array): the compiler then sees that the
  // in-flight direct loads into one buffer cannot alias reads of another and
  // does not drain them before every tile
  __shared__ __attribute__((aligned(16))) unsigned char tile0[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tile1[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tile2[kTileBytes];
  // slot table: the split's rows, two padding tiles, rounded up to whole
  // rounds of the workgroup so that every thread writes every round (no
  // branch for the compiler to sink the table loads into)
  constexpr int RMAX = (kMaxSplitRows + 2 * kRowsTile + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) int32_t sslot[RMAX * NT];
  __shared__ __attribute__((aligned(16))) float smask[RMAX * NT];  // 0 or -inf per row
  __shared__ __attribute__((aligned(16))) float4 xbuf[2 * NW * 4 * 64];   // partial S^T exchange, two parities
  // RS: latent scale of each row of the three tile buffers (0 for a row without an index)
  __shared__ __attribute__((aligned(16))) float tscl[RS ? 3 * kRowsTile : 4];

  // block -> (token, split, head part).  Workgroups are dispatched to the
  // eight XCDs round-robin (block b on XCD b % 8), so every workgroup of token
  // t is given a block on XCD t % 8: the head parts of a (token, split) share
  // the gathered rows through that XCD's L2, and the splits of a token share
  // its query rows.
  const int parts = a.H / (32 * HBW);
  const int bid = blockIdx.x;
  const int slot = bid >> 3;                   // ((t / 8) * splits + split) * parts + part
  const int part = slot % parts;
  const int split = (slot / parts) % a.splits;
  const int t = (slot / parts / a.splits) * 8 + (bid & 7);
  if (t >= a.s.T) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, nn = lane & 31;
  const int hbl = wave % HBW, ch = wave / HBW;   // head block in the workgroup, column (and depth) half
  const int partner = (1 - ch) * HBW + hbl;
  const int j0 = split * a.rows_per_split;
  int j1 = j0 + a.rows_per_split;
  j1 = j1 < a.K ? j1 : a.K;
  const int nrows = j1 > j0 ? j1 - j0 : 0;
  const int ntiles_split = (nrows + kRowsTile - 1) / kRowsTile;
  const int b = clampi(a.s.q_seq[t], 0, a.s.batch - 1);
  const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;
  const int32_t* irow = a.idx + (int64_t)t * a.K;
  const int head = (part * HBW + hbl) * 32 + nn;
  const unsigned char* kvb = (const unsigned char*)a.kv;

  // ---- gather: bf16 rows go global -> LDS directly --------------------------
  // wave instruction (row group rg, chunk group m) covers rows 8rg..8rg+7 and
  // chunks 8m..8m+7; lane L: row 8rg + L/8, chunk 8m + ((L%8) ^ swz(row)), so
  // that one 16-byte LDS write per lane fills 64 consecutive slots (1 KB).
  const int g_sub = lane & 7;
  constexpr int kRG = (4 + NW - 1) / NW;   // 8-row groups per wave

  // A pool below 4 GiB is addressed through a buffer descriptor (BUF): with a
  // global request in flight the compiler waits for every outstanding LDS read
  // before using any one of them, with a buffer request only for the one it
  // needs, so the operand prefetch keeps working while the gather flies.
  // Rows without a valid index are loaded as zeros (an offset past the
  // descriptor's range, or a zero row), so that whatever the pool holds in
  // the row they would otherwise read, they contribute exactly nothing.
  const uint32_t kv_bytes = (uint32_t)((uint64_t)a.s.num_pages * kPage * (kD * 2));  // BUF only
  const __amdgpu_buffer_rsrc_t kvrs = __builtin_amdgcn_make_buffer_rsrc((void*)kvb, 0, (int)kv_bytes, kRawBuffer);
  // source of lane's 16-byte piece of chunk group 0 of tile row r: a buffer
  // offset (BUF) or an address
  auto row_src = [&](int slot, int r) __attribute__((always_inline)) -> uint64_t {
    const uint32_t piece = 16 * (g_sub ^ swz(r));
    if constexpr (BUF)
      return slot >= 0 ? (uint64_t)slot * (kD * 2) + piece : (uint64_t)kv_bytes + piece;
    else
      return slot >= 0 ? (uint64_t)(uintptr_t)(kvb + (uint64_t)slot * (kD * 2) + piece)
                       : (uint64_t)(uintptr_t)((const unsigned char*)g_zero_kv_row + piece);
  };
  auto row_req = [&](uint64_t src, lds_u8* dst) __attribute__((always_inline)) {
    if constexpr (BUF)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kvrs, (lds_void*)dst, 16, (uint32_t)src, 0, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(uintptr_t)src,
                                       (lds_void*)dst, 16, 0, 0);
  };
  // one wave instruction fills the 64 consecutive 16-byte slots of (row group,
  // chunk group)
  auto issue_dma = [&](int i, lds_u8* dst) __attribute__((always_inline)) {
    const int32_t* ss = sslot + i * kRowsTile;
#pragma unroll
    for (int k = 0; k < kRG; ++k) {
      const int r = 8 * (wave + NW * k) + (lane >> 3);
      const uint64_t src = row_src(ss[r], r);
#pragma unroll
      for (int m = 0; m < 9; ++m) row_req(src + 128 * m, dst + 4096 * m + 1024 * (wave + NW * k));
    }
  };

  // ---- gather: fp8 rows go through registers and are dequantized to bf16 ----
  // thread -> row tid / TPR, 16-byte source chunks c = tid % TPR + TPR * m
  v4i stage[FP8 ? kFp8Loads : 1];
  float stage_scale[FP8 ? kFp8Loads : 1];
  const int f_row = tid / TPR, f_sub = tid % TPR;
  // fp8 pool and scales below 4 GiB (BUF): buffer descriptors, so that a row
  // without an index reads zeros from an offset past the range (no select, no
  // 64-bit address arithmetic per load)
  const uint32_t kv8_bytes = (uint32_t)((uint64_t)a.s.num_pages * kPage * 640);  // FP8 && BUF only
  const uint32_t sc_bytes = (uint32_t)(((uint64_t)a.s.num_pages * kPage * kDc >> (a.log2_scale_tokens + a.log2_scale_elems)) * 4);
  const __amdgpu_buffer_rsrc_t kv8rs = __builtin_amdgcn_make_buffer_rsrc((void*)kvb, 0, (int)kv8_bytes, kRawBuffer);
  const __amdgpu_buffer_rsrc_t scrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.kv_scale, 0, (int)sc_bytes, kRawBuffer);
  auto issue_fp8 = [&](int i) __attribute__((always_inline)) {
    const int32_t* ss = sslot + i * kRowsTile;
    const bool valid = ss[f_row] >= 0;  // otherwise zeros, whatever slot 0 holds
    const int slot = valid ? ss[f_row] : 0;
    // scale tile sizes are powers of two: shifts, not divisions, on the gather path
    const int page = slot >> 6, tok = slot & 63;
    const int lt = a.log2_scale_tokens, le = a.log2_scale_elems;
    const int64_t sbase = (((int64_t)page << (6 - lt)) + (tok >> lt)) << (9 - le);
    if constexpr (BUF) {
      const uint32_t row_off = valid ? (uint32_t)slot * 640u + 16u * f_sub : kv8_bytes;
      const uint32_t sc_off = valid ? (uint32_t)sbase * 4u : sc_bytes;
#pragma unroll
      for (int m = 0; m < kFp8Loads; ++m) {
        const int c = f_sub + TPR * m;
        stage[m] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(kv8rs, row_off, 16 * TPR * m, 0));
        if constexpr (!RS) {
          // latent chunks take their tile's scale, the rope chunks 1 (0 for a row without an index)
          const float sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(scrs, sc_off + 4u * ((16u * c) >> le), 0, 0));
          stage_scale[m] = c < 32 ? sc : (valid ? 1.f : 0.f);
        }
      }
      // RS: the row's one latent scale (0 past the range)
      if constexpr (RS) stage_scale[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(scrs, sc_off, 0, 0));
    } else {
      const unsigned char* src = kvb + (int64_t)slot * 640 + 16 * f_sub;
#pragma unroll
      for (int m = 0; m < kFp8Loads; ++m) {
        const int c = f_sub + TPR * m;
        const v4i v = *(const v4i*)(src + 16 * TPR * m);
        stage[m] = valid ? v : v4i{0, 0, 0, 0};
        if constexpr (!RS) {
          const float sc = c < 32 ? a.kv_scale[sbase + ((16 * c) >> le)] : 1.f;
          stage_scale[m] = valid ? sc : 0.f;
        }
      }
      if constexpr (RS) stage_scale[0] = valid ? a.kv_scale[sbase] : 0.f;
    }
  };
  auto commit_fp8 = [&](lds_u8* dst, float* sdst) __attribute__((always_inline)) {
    const int r = f_row, sw = swz(r);
    if constexpr (RS) {
      if (f_sub == 0) sdst[r] = stage_scale[0];
    }
#pragma unroll
    for (int m = 0; m < kFp8Loads; ++m) {
      const int c = f_sub + TPR * m;
      const v4i v = stage[m];
      if (c < 32) {
        uint32_t o[8];
        if constexpr (RS) {
          // exact conversion, two codes per instruction (scale operand 1)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[w], 1.f, false));
            o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[w], 1.f, true));
          }
        } else {
          const float sc = stage_scale[m];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float2 f0 = fp8x2_to_f32<false>((uint32_t)v[w]);
            const float2 f1 = fp8x2_to_f32<true>((uint32_t)v[w]);
            o[2 * w] = pack_bf16x2(f0.x * sc, f0.y * sc);
            o[2 * w + 1] = pack_bf16x2(f1.x * sc, f1.y * sc);
          }
        }
        const int c0 = 2 * c, c1 = 2 * c + 1;
        *(lds_v4i*)(dst + ((c0 >> 3) * 256 + r * 8 + ((c0 & 7) ^ sw)) * 16) =
            v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
        *(lds_v4i*)(dst + ((c1 >> 3) * 256 + r * 8 + ((c1 & 7) ^ sw)) * 16) =
            v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
      } else {
        const int cr = 64 + (c - 32);
        *(lds_v4i*)(dst + ((cr >> 3) * 256 + r * 8 + ((cr & 7) ^ sw)) * 16) = v;
      }
    }
  };

  v8bf qb[kHalfSteps];
  // physical slots of all rows of this split (-1: no row).  The index loads go
  // out first, then the query loads, then the page-table loads: loads complete
  // in order, so the page-table loads wait only for the indices, and the
  // query's 72 KB arrive while the table is resolved.
  // Tiles past the split's last valid row hold only padding (a causal row
  // with fewer visible positions than K ends in -1s): they would contribute
  // exactly nothing, so the loop stops at the last tile with a valid row.
  __shared__ int s_last[NW];
  int last_ok = -1;
  {
    const int rows = (ntiles_split + 2) * kRowsTile;
    // loads are unconditional (clamped indices) so that none waits for another
    int pos[RMAX];
#pragma unroll
    for (int u = 0; u < RMAX; ++u) {
      const int j = j0 + tid + NT * u;
      pos[u] = irow[j < a.K ? j : a.K - 1];
    }
    // query operand: Q^T[depth, head], lane (hh, nn): head nn.  The wave's
    // step j is global step st = 4(j/2) + 2ch + j%2, i.e. 16-byte chunk 2st + hh.
    const v8bf* qr = (const v8bf*)((const uint16_t*)a.q + ((int64_t)t * a.H + head) * kD);
#pragma unroll
    for (int j = 0; j < kHalfSteps; ++j) qb[j] = qr[2 * (4 * (j >> 1) + 2 * ch + (j & 1)) + hh];
    int page[RMAX];
#pragma unroll
    for (int u = 0; u < RMAX; ++u) {
      const int p = pos[u];
      page[u] = table[(p >= 0 && p < a.s.max_visible ? p : 0) >> 6];
    }
#pragma unroll
    for (int u = 0; u < RMAX; ++u) {
      const int r = tid + NT * u, p = pos[u];
      const bool ok = r < rows && j0 + r < j1 && p >= 0 && p < a.s.max_visible;
      const int pg = clampi(page[u], 0, a.s.num_pages - 1);
      sslot[r] = ok ? pg * kPage + (p & (kPage - 1)) : -1;
      smask[r] = ok ? 0.f : -INFINITY;
      // the wave's last valid row of this round, from one ballot (scalar)
      const uint64_t bm = __builtin_amdgcn_ballot_w64(ok);
      if (bm) last_ok = NT * u + 64 * wave + 63 - __builtin_clzll(bm);
    }
  }
  if (lane == 0) s_last[wave] = last_ok;
  // keep the query operand resident: without this the compiler re-loads it
  // from memory inside the tile loop to save registers
#pragma unroll
  for (int j = 0; j < kHalfSteps; ++j) asm volatile("" : "+v"(qb[j]));

  // per-lane LDS read bases (see the layout note above)
  //  S^T A operand, global step st = 4k + mm: chunk 2st + hh -> group k, in-group
  //  2mm + hh; the wave's steps have mm = 2ch + j%2 and k = j/2
  int sbase[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) sbase[x] = 16 * (nn * 8 + ((2 * (2 * ch + x) + hh) ^ swz(nn)));
  //  V^T A operand via transposing reads: source lane s' = lane%16 gives row
  //  offset jrow = s'/4 and vcol quad qd = s'%4; lane group g = lane/16.
  const int g = lane >> 4, sp = lane & 15, jrow = sp >> 2, qd = sp & 3;
  const int vrow0 = 4 * (g >> 1) + jrow;            // + 8a + 16mf
  // one base per (column parity, a); the swizzle is the same for mf = 0, 1
  int vbase[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      const int vr = vrow0 + 8 * aa;
      vbase[par][aa] = 128 * vr + 16 * ((4 * par + 2 * (g & 1) + (qd >> 1)) ^ swz(vr)) + 8 * (qd & 1) +
                       4096 * 4 * ch;      // column half: chunk groups 4..7
    }

  // Softmax reference: p = 2^(l - m_ref) with one fixed m_ref per head, the
  // largest logit of the first tile that has a valid row, so no tile rescales
  // the accumulator.  m_ref never exceeds the true maximum, so nothing that
  // matters underflows; if a later tile's logits exceed m_ref by more than
  // 2^100 (which could overflow the fp32 sums), the workgroup runs its rows
  // once more with m_ref = the maximum seen over all of them.
  v16f o[kVT];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
  bool overflow = false;

  lds_u8* const T0 = (lds_u8*)tile0;
  lds_u8* const T1 = (lds_u8*)tile1;
  lds_u8* const T2 = (lds_u8*)tile2;
  // RS: the row-scale array of a tile buffer (resolved at compile time: the
  // buffers are passed as the constants above)
  auto scl_of = [&](lds_u8* b) __attribute__((always_inline)) -> float* {
    if constexpr (RS) return tscl + kRowsTile * (b == T0 ? 0 : (b == T1 ? 1 : 2));
    return tscl;
  };
  __syncthreads();
  int last = s_last[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) last = max(last, s_last[w]);
  // tiles up to the one holding row `last`, in a scalar register (the same in
  // every lane), so that the tile loop keeps scalar control
  const int ntiles = __builtin_amdgcn_readfirstlane((last + kRowsTile) / kRowsTile);
  {
  // ---- software-pipelined tiles ------------------------------------
  // Iteration i requests tile i+2 into the buffer tile i-1 used, computes the
  // partial scores of tile i+1 while the softmax of tile i runs between its
  // MFMAs (starting with the read of the partner's half of tile i), then
  // O += V^T P^T for tile i, writes its half of tile i+1, and ends with the
  // one barrier that publishes tile i+2 and the partial scores of tile i+1.  bf16 rows go
  // straight into LDS; fp8 rows are loaded into registers at the start of the
  // iteration and dequantized into the buffer after the output MFMAs.
  // Requests and score passes past the last tile run on the slot table's -1
  // padding (zero rows) and their results are never used; this keeps the loop
  // free of conditional requests, which would make the compiler drain every
  // load before each read.
  // additive masks of this lane's 16 rows of tile i (rows 8k + 4hh + 0..3
  // are four consecutive entries)
  struct Flags {
    float4 f[4];
  };
  auto load_flags = [&](int i) __attribute__((always_inline)) -> Flags {
    const float* sm = smask + i * kRowsTile;
    Flags fl;
#pragma unroll
    for (int k = 0; k < 4; ++k) fl.f[k] = *(const float4*)(sm + 8 * k + 4 * hh);
    return fl;
  };
  // operands are read PF steps ahead of their MFMA: LDS latency is about six
  // MFMA issue slots
  constexpr int PF = 6, PFV = 6;
  // partial S^T of the tile in `buf` over this wave's half of the depth;
  // between(j) runs after the MFMA of step j
  // RS: the wave's last two steps are rope depth (global steps 32 + 2ch and
  // 33 + 2ch); they accumulate apart, and the partial is s * latent + rope
  // with the scales `scl` of the tile's rows
  auto s_partial = [&](lds_u8* buf, const float* scl, auto&& between) __attribute__((always_inline)) -> v16f {
    v16f acc = v16f{};
    v16f accr = v16f{};
    v8bf kring[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) kring[j] = *(lds_v8bf*)(buf + sbase[j & 1] + 4096 * (j >> 1));
#pragma unroll
    for (int j = 0; j < kHalfSteps; ++j) {
      const v8bf kf = kring[j % PF];
      if (j + PF < kHalfSteps) kring[j % PF] = *(lds_v8bf*)(buf + sbase[(j + PF) & 1] + 4096 * ((j + PF) >> 1));
      if (RS && j >= kHalfSteps - 2)
        accr = mfma_bf16(kf, qb[j], accr);
      else
        acc = mfma_bf16(kf, qb[j], acc);
      between(j);
    }
    if constexpr (RS) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 s4 = *(const float4*)(scl + 8 * k + 4 * hh);
        acc[4 * k] = fmaf(s4.x, acc[4 * k], accr[4 * k]);
        acc[4 * k + 1] = fmaf(s4.y, acc[4 * k + 1], accr[4 * k + 1]);
        acc[4 * k + 2] = fmaf(s4.z, acc[4 * k + 2], accr[4 * k + 2]);
        acc[4 * k + 3] = fmaf(s4.w, acc[4 * k + 3], accr[4 * k + 3]);
      }
    }
    return acc;
  };
  auto xwrite = [&](const v16f& acc, int par) __attribute__((always_inline)) {
    float4* mine = xbuf + (par * NW + wave) * 256 + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) mine[64 * k] = make_float4(acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]);
  };
  // both waves of a head block add the same two fp32 values: identical S^T.
  // The partner's half is read as the next iteration's score MFMAs start, so
  // the read's latency runs beside them.
  auto xload = [&](float4 (&xo)[4], int par) __attribute__((always_inline)) {
    const float4* other = xbuf + (par * NW + partner) * 256 + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) xo[k] = other[64 * k];
  };
  auto xadd = [&](v16f& acc, const float4 (&xo)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[4 * k] += xo[k].x;
      acc[4 * k + 1] += xo[k].y;
      acc[4 * k + 2] += xo[k].z;
      acc[4 * k + 3] += xo[k].w;
    }
  };
  v16f sacc;   // this wave's half of S^T of the tile the next iteration finishes
  // gather of tile i+2: source rows first, then every 16-byte request right
  // after the first score MFMA (issued together, they land earlier than when
  // spread over the score steps)
  auto dma_src = [&](int i, int k) __attribute__((always_inline)) -> uint64_t {
    const int r = 8 * (wave + NW * k) + (lane >> 3);
    return row_src(sslot[i * kRowsTile + r], r);
  };
  auto dma_one = [&](uint64_t src, lds_u8* dst, int k, int m) __attribute__((always_inline)) {
    row_req(src + 128 * m, dst + 4096 * m + 1024 * (wave + NW * k));
  };
  auto iter = [&](int i, lds_u8* cur, lds_u8* nxt, lds_u8* fut) __attribute__((always_inline)) {
    uint64_t dsrc[kRG];
    if constexpr (FP8) {
      issue_fp8(i + 2);  // into registers; dequantized into LDS after the output MFMAs
    } else {
#pragma unroll
      for (int k = 0; k < kRG; ++k) dsrc[k] = dma_src(i + 2, k);
    }
    const Flags fl = load_flags(i);
    // RS: the latent scales of tile i's rows go onto their weights in P
    Flags rsc{};
    if constexpr (RS) {
#pragma unroll
      for (int k = 0; k < 4; ++k) rsc.f[k] = *(const float4*)(scl_of(cur) + 8 * k + 4 * hh);
    }
    // softmax of tile i (log2 domain; lane owns head nn, rows 8(r/4) + 4hh + r%4).
    // The maximum over both lane halves (one v_permlane32_swap) is needed only
    // until m_ref is set; afterwards each lane tracks its own maximum, for the
    // overflow test and the second pass, and p = 2^(s * scale - m_ref) is one
    // FMA and one exp (invalid rows hold -inf and give 0).
    float sv[16];
    float tloc = -INFINITY, psum = 0.f, mneg = 0.f;
    v8bf pb[2];
    float4 xo[4];
    auto soft = [&](int j) __attribute__((always_inline)) {
      if constexpr (!FP8) {
        if (j == 0) {
#pragma unroll
          for (int d = 0; d < kRG * 9; ++d) dma_one(dsrc[d / 9], fut, d / 9, d % 9);
        }
      }
      if (j == 0) {
        xload(xo, i & 1);   // the partner's half of tile i, published by the last barrier
      } else if (j == 2) {
        xadd(sacc, xo);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float4 f = fl.f[r >> 2];
          sv[r] = sacc[r] + ((r & 3) == 0 ? f.x : (r & 3) == 1 ? f.y : (r & 3) == 2 ? f.z : f.w);
          tloc = fmaxf(tloc, sv[r]);
        }
      } else if (j == 3) {
        tloc *= a.scale_log2;  // the scale is positive
        m_seen = fmaxf(m_seen, tloc);
        if (__builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tloc), __float_as_uint(tloc), false, false);
          const float both = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          if (m_ref == -INFINITY) m_ref = both;
        }
        overflow |= tloc > m_ref + 100.f;
        mneg = m_ref == -INFINITY ? -INFINITY : -m_ref;   // no valid row yet: every p is 0
      } else if (j >= 4 && j < 12) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int r = 2 * (j - 4) + rr;
          const float pv = fast_exp2(fmaf(sv[r], a.scale_log2, mneg));
          psum += pv;
          if constexpr (RS) {
            const float4 f = rsc.f[r >> 2];
            const float rs = (r & 3) == 0 ? f.x : (r & 3) == 1 ? f.y : (r & 3) == 2 ? f.z : f.w;
            pb[r >> 3][r & 7] = static_cast<__bf16>(pv * rs);
          } else {
            pb[r >> 3][r & 7] = static_cast<__bf16>(pv);
          }
        }
      }
    };
    v16f snext = s_partial(nxt, scl_of(nxt), soft);
    // O^T += V^T . P^T for tile i; MFMA mf covers tile rows 16mf + R(hh, jj)
    auto vfrag = [&](int vt, int mf) -> v8bf {
      const int imm = 4096 * (vt >> 1) + 2048 * mf;
      const v4bf x0 = lds_tr16(cur, vbase[vt & 1][0] + imm);
      const v4bf x1 = lds_tr16(cur, vbase[vt & 1][1] + imm);
      return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    v8bf vring[PFV];
#pragma unroll
    for (int k = 0; k < PFV; ++k) vring[k] = vfrag(k % kVT, k / kVT);
#pragma unroll
    for (int k = 0; k < 2 * kVT; ++k) {
      const int vt = k % kVT, mf = k / kVT;
      const v8bf af = vring[k % PFV];
      if (k + PFV < 2 * kVT) vring[k % PFV] = vfrag((k + PFV) % kVT, (k + PFV) / kVT);
      o[vt] = mfma_bf16(af, pb[mf], o[vt]);
    }
    // the partial scores of tile i+1 go out after the output MFMAs are issued:
    // by then the score chain has finished, so the writes do not wait for it
    xwrite(snext, (i + 1) & 1);
    if constexpr (FP8) commit_fp8(fut, scl_of(fut));  // tile i+2: buffer free since the last barrier
    l_run += psum;
    // tile i+2 is in LDS and the partial scores of tile i+1 are published
    wait_vm_lgkm0<0>();
    asm volatile("s_barrier" ::: "memory");
    sacc = snext;
  };
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int v = 0; v < kVT; ++v) o[v] = v16f{};
    l_run = 0.f;
    overflow = false;
    if (pass == 1) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m_seen), __float_as_uint(m_seen), false, false);
      m_ref = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // prologue: tiles 0 and 1 in LDS, full scores of tile 0
    if constexpr (FP8) {
      issue_fp8(0);
      commit_fp8(T0, scl_of(T0));
      issue_fp8(1);
      commit_fp8(T1, scl_of(T1));
    } else {
      issue_dma(0, T0);
      issue_dma(1, T1);
    }
    wait_vm_lgkm0<0>();
    asm volatile("s_barrier" ::: "memory");
    // this wave's half of the scores of tile 0; iteration 0 adds the partner's
    sacc = s_partial(T0, scl_of(T0), [](int) {});
    xwrite(sacc, 0);
    wait_vm_lgkm0<63>();
    asm volatile("s_barrier" ::: "memory");
    int i = 0;
    for (; i + 3 <= ntiles; i += 3) {
      iter(i, T0, T1, T2);
      iter(i + 1, T1, T2, T0);
      iter(i + 2, T2, T0, T1);
    }
    if (i < ntiles) iter(i, T0, T1, T2);
    if (i + 1 < ntiles) iter(i + 1, T1, T2, T0);
    // every wave agrees on a second pass; the barrier also retires this pass's tiles
    if (!__syncthreads_or(overflow)) break;
  }
  }

  // ---- finish: normalise, stage the workgroup's heads x 512 columns in LDS
  // (the tiles are free after the pass loop's last barrier), then write each
  // head's row with contiguous 16-byte stores, one whole 1 KB row per wave
  // store instruction.  Stored straight from the accumulator, a store
  // instruction would touch 32 head rows 1 KB apart with 8 bytes each.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_ref + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  constexpr int kPitch = kDc * 2 + 16;           // staged row bytes; the pad keeps LDS writes to 2-way conflicts
  static_assert(32 * kPitch <= kTileBytes, "a head block's rows fit one tile buffer");
  {
    lds_u8* srow = (hbl == 0 ? T0 : T1) + nn * kPitch + 2 * (kVH * ch);
#pragma unroll
    for (int vt = 0; vt < kVT; ++vt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int vc = 32 * vt + 8 * q4 + 4 * hh;
        const uint64_t w = (uint64_t)pack_bf16x2(o[vt][4 * q4] * inv, o[vt][4 * q4 + 1] * inv) |
                           ((uint64_t)pack_bf16x2(o[vt][4 * q4 + 2] * inv, o[vt][4 * q4 + 3] * inv) << 32);
        *(__attribute__((address_space(3))) uint64_t*)(srow + 2 * vc) = w;
      }
  }
  __syncthreads();
  uint16_t* obase = a.splits == 1 ? (uint16_t*)a.out + (int64_t)t * a.H * kDc
                                  : a.ws_o + ((int64_t)t * a.splits + split) * a.H * kDc;
  const int head0 = part * HBW * 32;
  constexpr int kRowChunks = kDc * 2 / 16;       // 16-byte chunks per output row
#pragma unroll 4
  for (int c = tid; c < HBW * 32 * kRowChunks; c += NT) {
    const int r = c / kRowChunks, k = c % kRowChunks;
    const v4i v = *(const lds_v4i*)((r < 32 ? T0 : T1) + (r & 31) * kPitch + 16 * k);
    *(v4i*)(obase + (int64_t)(head0 + r) * kDc + 8 * k) = v;
  }
  if (hh == 0 && ch == 0) {
    if (a.splits == 1) {
      if (a.lse) a.lse[(int64_t)t * a.H + head] = lse_v;
    } else {
      a.ws_lse[((int64_t)t * a.splits + split) * a.H + head] = lse_v;
    }
  }
}

// Merge split partials: out = sum_s exp(lse_s - LSE) * O_s, in split order.
// One wave per (token, head), eight output columns per lane.  Every load of a
// group of kCombineGroup splits is issued before the first result is used (the
// split LSEs lane-parallel, one split per lane), so a merge of up to four
// splits waits on memory once instead of twice per split.
constexpr int kCombineGroup = 4;
constexpr int kMaxSplits = 32;  // mla_splits never returns more; one LSE per lane

__global__ __launch_bounds__(256) void k_mla_combine(MlaArgs a) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (h >= a.H) return;
  const int S = a.splits;
  const int64_t hstride = (int64_t)a.H * kDc;  // between the partials of consecutive splits
  const float* __restrict__ lse_t = a.ws_lse + (int64_t)t * S * a.H + h;
  const uint16_t* __restrict__ o_t = a.ws_o + ((int64_t)t * S * a.H + h) * kDc + lane * 8;

  const float ls = lane < S ? lse_t[(int64_t)lane * a.H] : -INFINITY;
  uint4 v[kCombineGroup];
  auto load_group = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u)
      if (g + u < S) v[u] = *reinterpret_cast<const uint4*>(o_t + (g + u) * hstride);
  };
  load_group(0);
  const float mx = wave_max(ls);  // exact, so every lane holds the same value
  const float wl = mx == -INFINITY ? 0.f : __expf(ls - mx);

  float tot = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < S; g += kCombineGroup) {
    if (g > 0) load_group(g);
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      if (g + u >= S) break;
      const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), g + u));
      tot += wgt;
      if (wgt != 0.f) {
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = fmaf(wgt, __uint_as_float(wd[k] << 16), acc[2 * k]);
          acc[2 * k + 1] = fmaf(wgt, __uint_as_float(wd[k] & 0xffff0000u), acc[2 * k + 1]);
        }
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint16_t* out = (uint16_t*)a.out + ((int64_t)t * a.H + h) * kDc + lane * 8;
  uint4 w;
  w.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  w.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  w.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *(uint4*)out = w;
  if (a.lse && lane == 0) a.lse[(int64_t)t * a.H + h] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
}

int mla_splits(int T, int K, int heads) {
  if (T <= 0) return 1;
  const int cus = num_cus();
  const int parts = heads >= 128 ? 2 : 1;  // workgroups per (token, split)
  int s = (cus / parts + T - 1) / T;       // about one workgroup per CU
  const int min_s = (K + kMaxSplitRows - 1) / kMaxSplitRows;   // a split holds at most kMaxSplitRows rows
  const int max_s = (K + kRowsTile * 2 - 1) / (kRowsTile * 2);  // keep >= 2 tiles per split
  s = s > max_s ? max_s : s;
  s = s > kMaxSplits ? kMaxSplits : s;
  s = s < min_s ? min_s : s;
  return s < 1 ? 1 : s;
}

size_t mla_workspace_bytes(int T, int K, int heads, int latent) {
  const int s = mla_splits(T, K, heads);
  if (s <= 1) return 0;
  // bf16 partial outputs, then one float LSE per (token, split, head)
  return (size_t)T * s * heads * ((size_t)latent * sizeof(uint16_t) + sizeof(float)) + 256;
}

hipError_t launch_sparse_mla(const void* q, int heads, const sia_kv_in& kv, const SeqArgs& s, const int32_t* idx,
                             int K, float scale, void* out, float* lse, int splits, void* ws, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  MlaArgs a{};
  a.q = q;
  a.kv = kv.kv_pool;
  a.kv_scale = kv.kv_scale;
  a.scale_tokens = kv.scale_tokens;
  a.scale_elems = kv.scale_elems;
  a.log2_scale_tokens = __builtin_ctz((unsigned)(kv.scale_tokens > 0 ? kv.scale_tokens : 1));
  a.log2_scale_elems = __builtin_ctz((unsigned)(kv.scale_elems > 0 ? kv.scale_elems : 1));
  a.H = heads;
  a.Dc = kv.latent_dim;
  a.Dr = kv.rope_dim;
  a.s = s;
  a.idx = idx;
  a.K = K;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  if (kv.dtype == SIA_F32) {
    a.splits = 1;
    hipLaunchKernelGGL(k_sparse_mla_f32, dim3(s.T, heads), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  a.splits = splits < 1 ? 1 : splits;
  if (a.splits > kMaxSplits) return hipErrorInvalidValue;
  int rps = (K + a.splits - 1) / a.splits;
  rps = (rps + kRowsTile - 1) / kRowsTile * kRowsTile;
  a.rows_per_split = rps;
  if (a.splits > 1) {
    a.ws_o = (uint16_t*)ws;
    a.ws_lse = (float*)(a.ws_o + (size_t)s.T * a.splits * heads * kDc);
  }
  const int64_t units = ((int64_t)(s.T + 7) / 8) * a.splits;   // per XCD
  const int parts = heads >= 128 ? 2 : 1;
  const int64_t nblocks = units * parts * 8;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblocks);
  const bool fp8 = kv.dtype == SIA_FP8_E4M3;
  // bf16 pools that buffer offsets (32 bits) can address take the buffer form
  // (with room past the end for the zero-row offsets)
  const bool buf = (uint64_t)s.num_pages * kPage * (kD * 2) <= 0xfffff000ull;
  // fp8 rows are 640 bytes; the scale array must fit a descriptor too
  const uint64_t sc_entries = ((uint64_t)s.num_pages * kPage * kDc) >> (a.log2_scale_tokens + a.log2_scale_elems);
  const bool buf8 = (uint64_t)s.num_pages * kPage * 640 <= 0xfffff000ull && sc_entries * 4 <= 0xfffff000ull;
  // one latent scale per row (tiles of 512 elements): the scale goes onto scores and P
  const bool rs = kv.scale_elems == kDc;
#define SIA_LAUNCH_MLA(NW)                                                                         \
  if (fp8 && buf8 && rs)                                                                           \
    hipLaunchKernelGGL((k_sparse_mla_mfma<NW, true, true, true>), grid, dim3(NW * 64), 0, st, a);  \
  else if (fp8 && buf8)                                                                            \
    hipLaunchKernelGGL((k_sparse_mla_mfma<NW, true, true>), grid, dim3(NW * 64), 0, st, a);        \
  else if (fp8 && rs)                                                                              \
    hipLaunchKernelGGL((k_sparse_mla_mfma<NW, true, false, true>), grid, dim3(NW * 64), 0, st, a); \
  else if (fp8)                                                                                    \
    hipLaunchKernelGGL((k_sparse_mla_mfma<NW, true, false>), grid, dim3(NW * 64), 0, st, a);       \
  else if (buf)                                                                              \
    hipLaunchKernelGGL((k_sparse_mla_mfma<NW, false, true>), grid, dim3(NW * 64), 0, st, a); \
  else                                                                                       \
    hipLaunchKernelGGL((k_sparse_mla_mfma<NW, false, false>), grid, dim3(NW * 64), 0, st, a);
  if (heads >= 64) {
    SIA_LAUNCH_MLA(4)
  } else {
    SIA_LAUNCH_MLA(2)
  }
#undef SIA_LAUNCH_MLA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(k_mla_combine, dim3(s.T, (heads + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sia

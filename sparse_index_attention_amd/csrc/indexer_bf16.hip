// Step 1, bfloat16 path — indexer scores from bf16 queries and keys, no
// scales: the indexer's precision path for prefill and decode [P2] "Efficient
// Inference Deployment and Optimization for Hybrid Attention LLMs", section
// 3.2; [P5] "Inference Adaptation and Performance Optimization for a
// Domestically Developed LLM's New Architecture", section 3.1.
//
//   score[t, s] = sum_h w[t,h] * ReLU(<q[t,h], k[s]>),  s <= q_pos[t]
//
// The contraction runs on v_mfma_f32_32x32x16_bf16 (8 K steps over dim 128).
// Structure as in the fp8 prefill kernel: a workgroup takes 4 consecutive
// queries (one per wave) and a chunk of pages; each 16 KB key page goes
// global -> registers (two pages ahead) -> a double-buffered LDS page that the
// waves of its sequence read as their B operand.  The chunk length adapts to
// the batch so that decode (one query per sequence) still fills the GPU.
#include "block_prims.hpp"
#include "index_core.hpp"

namespace sia {

namespace {

constexpr int kBQ = 4;                 // queries (waves) per workgroup
constexpr int kBThreads = 64 * kBQ;
constexpr int kBMaxChunk = 128;        // pages per work item, at most
constexpr int kBRow = 256;             // bytes of a bf16 key row

// 16-byte chunk j (0..15) of key row r sits at chunk j ^ (r & 15): the 16 lanes
// of one read phase (rows r..r+15, same j) cover all 64 banks.
__device__ __forceinline__ int bswz(int r, int j) { return r * kBRow + 16 * (j ^ (r & 15)); }

__device__ __forceinline__ v16f mfma_bf16x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct BStage {  // one thread's 64 bytes of a key page in flight
  uint4 v[4];
};

// Lane l: nn = l % 32 (head within an M tile / key within an N tile), hh = l / 32.
// K step st of lane half hh covers depth [16st + 8hh, +8) = row bytes
// [32st + 16hh, +16), i.e. 16-byte chunk 2st + hh (same for both operands).
template <int HI>
__global__ __launch_bounds__(kBThreads, 2) void k_index_scores_bf16(IndexArgs a, int n_qblocks, int chunk) {
  constexpr int MT = HI / 32;
  __shared__ __attribute__((aligned(16))) uint8_t kl[2][kPage * kBRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, nn = lane & 31;
  const int ch = (int)blockIdx.x / n_qblocks;
  const int t0 = (n_qblocks - 1 - (int)blockIdx.x % n_qblocks) * kBQ;

  const int nq = min(kBQ, a.s.T - t0);
  int qseq[kBQ], cvis[kBQ], cmax = 0;
#pragma unroll
  for (int i = 0; i < kBQ; ++i) {
    qseq[i] = i < nq ? clampi(a.s.q_seq[t0 + i], 0, a.s.batch - 1) : -1;
    cvis[i] = i < nq ? (clampi(a.s.q_pos[t0 + i], -1, a.s.max_visible - 1) >> 6) + 1 : 0;
    cmax = max(cmax, cvis[i]);
  }
  const int c_begin = ch * chunk;
  if (c_begin >= cmax) return;

  const int t = t0 + wave;
  const bool has_q = wave < nq;
  const int pos = has_q ? clampi(a.s.q_pos[t], -1, a.s.max_visible - 1) : -1;
  const int my_seq = has_q ? clampi(a.s.q_seq[t], 0, a.s.batch - 1) : -1;
  const int c_own = (pos >> 6) + 1;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + (int64_t)(has_q ? t : 0) * a.ld, 0, a.s.max_visible * 4, kRawBuffer);
  const uint8_t* __restrict__ kpool = (const uint8_t*)a.k_pool;
  const int sr = tid >> 2, sj = 4 * (tid & 3);  // thread moves row sr, chunks sj .. sj+3

  // this wave's query (operand A) and head weights
  v8bf qa[MT][8];
  float wr[MT][16];
  if (has_q) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* qr = (const uint8_t*)a.q + ((int64_t)t * HI + 32 * mt + nn) * kBRow + 16 * hh;
#pragma unroll
      for (int st = 0; st < 8; ++st) qa[mt][st] = *(const v8bf*)(qr + 32 * st);
#pragma unroll
      for (int r = 0; r < 16; ++r) wr[mt][r] = a.w[(int64_t)t * HI + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3)];
    }
  }

  auto compute = [&](int c, int cur) __attribute__((always_inline)) {
    float p[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = 32 * kt + nn;
      v8bf kb[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) kb[st] = *(const v8bf*)&kl[cur][bswz(r, 2 * st + hh)];
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v16f acc = {};
#pragma unroll
        for (int st = 0; st < 8; ++st) acc = mfma_bf16x16(qa[mt][st], kb[st], acc);
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) sum = fmaf(wr[mt][r2], __int_as_float(max(__float_as_int(acc[r2]), 0)), sum);
      }
      p[kt] = sum;
    }
    // lanes l and l+32 hold the two head halves of keys l and 32+l
    const auto hv = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
    float score = __uint_as_float(hv[0]) + __uint_as_float(hv[1]);
    if (c * 64 + 63 > pos) score = c * 64 + lane > pos ? -INFINITY : score;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), srs, (c * 64 + lane) * 4, 0, 0);
  };

  for (int i = 0; i < nq; ++i) {
    int b = -1;
#pragma unroll
    for (int j = 0; j < kBQ; ++j) b = j == i ? qseq[j] : b;
    b = __builtin_amdgcn_readfirstlane(b);
    bool seen = false;
    int ce = 0;
#pragma unroll
    for (int j = 0; j < kBQ; ++j) {
      seen = seen || (j < i && qseq[j] == b);
      ce = qseq[j] == b ? max(ce, cvis[j]) : ce;
    }
    if (seen) continue;
    const int c_end = min(c_begin + chunk, __builtin_amdgcn_readfirstlane(ce));
    if (c_begin >= c_end) continue;
    const bool mine = my_seq == b;

    const int32_t* table = a.s.block_table + (int64_t)b * a.s.max_pages;
    int pg[kBMaxChunk / 64];
#pragma unroll
    for (int k = 0; k < kBMaxChunk / 64; ++k)
      pg[k] = clampi(table[min(c_begin + 64 * k + lane, c_end - 1)], 0, a.s.num_pages - 1);
    auto gload = [&](int c) __attribute__((always_inline)) {
      const int o = min(c, c_end - 1) - c_begin;
      const int page = __builtin_amdgcn_readlane(o >> 6 ? pg[1] : pg[0], o & 63);
      const uint8_t* src = kpool + (int64_t)page * (kPage * kBRow) + sr * kBRow + 16 * sj;
      BStage g;
#pragma unroll
      for (int k = 0; k < 4; ++k) g.v[k] = *(const uint4*)(src + 16 * k);
      return g;
    };
    auto lwrite = [&](int buf, const BStage& g) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 4; ++k) *(uint4*)&kl[buf][bswz(sr, sj + k)] = g.v[k];
    };
    BStage sa = gload(c_begin), sb = gload(c_begin + 1);
    __syncthreads();  // the previous round's reads of both buffers are done
    lwrite(0, sa);
    sa = gload(c_begin + 2);
    int c = c_begin;
    for (; c + 2 <= c_end; c += 2) {
      __syncthreads();
      lwrite(1, sb);
      sb = gload(c + 3);
      if (mine && c < c_own) compute(c, 0);
      __syncthreads();
      lwrite(0, sa);
      sa = gload(c + 4);
      if (mine && c + 1 < c_own) compute(c + 1, 1);
    }
    if (c < c_end) {
      __syncthreads();
      if (mine && c < c_own) compute(c, 0);
    }
  }
}

}  // namespace

hipError_t launch_index_scores_bf16(const sia_indexer_in& in, const SeqArgs& s, float* scores, int64_t ld,
                                    hipStream_t st) {
  const IndexArgs a = index_args(in, s, scores, ld);
  if (s.T == 0 || s.max_visible == 0) return hipSuccess;
  if (s.max_visible > (1 << 29)) return hipErrorInvalidValue;
  const int n_pages = (s.max_visible + 63) / 64;
  const int nqb = (s.T + kBQ - 1) / kBQ;
  // pages per item: whole 128-page chunks when there are many query blocks,
  // shorter ones so that decode-sized batches still give every CU work
  const int64_t want = 2LL * num_cus();
  int chunk = (int)(((int64_t)n_pages * nqb + want - 1) / want);
  chunk = chunk < 4 ? 4 : (chunk > kBMaxChunk ? kBMaxChunk : chunk);
  const int64_t grid = (int64_t)nqb * ((n_pages + chunk - 1) / chunk);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (in.heads == 64)
    hipLaunchKernelGGL(k_index_scores_bf16<64>, dim3((unsigned)grid), dim3(kBThreads), 0, st, a, nqb, chunk);
  else
    hipLaunchKernelGGL(k_index_scores_bf16<32>, dim3((unsigned)grid), dim3(kBThreads), 0, st, a, nqb, chunk);
  return hipGetLastError();
}

}  // namespace sia

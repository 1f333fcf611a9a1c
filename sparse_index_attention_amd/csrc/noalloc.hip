// Allocation-free form of the fused call (sia_index_select_attend_noalloc),
// for callers that cannot allocate device memory: code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc.
//
// The workspace is a file-scope device array of kNoAllocScratchBytes, one copy
// per GPU, held until the process ends.  Its device address is looked up once
// per device with hipGetSymbolAddress (the array's name in host code is only a
// host-side stand-in) and handed to the same kernels as the caller-provided
// workspace of sia_index_select_attend.  No kernel of that path needs its
// workspace cleared, so nothing is reset between calls; calls that overlap on
// one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sia_internal.hpp"

namespace sia {

constexpr size_t kNoAllocScratchBytes = SIA_NOALLOC_WORKSPACE_BYTES;  // 64 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call made on that device.
static hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sia

extern "C" {

int sia_index_select_attend_noalloc(const sia_indexer_in* in, const void* q_mla, sia_dtype q_dtype, int32_t heads,
                                    const sia_kv_in* kv, const sia_seqmap* seq, int32_t K, int32_t order,
                                    float softmax_scale, int32_t* idx_out, void* out, float* lse,
                                    hipStream_t stream) {
  const size_t need =
      sia_workspace_size(SIA_OP_INDEX_SELECT_ATTEND, seq, K, heads, kv ? kv->latent_dim : 0);
  // Invalid arguments, empty batches and workspaces beyond the array's size go
  // through the regular entry point without a workspace: it validates every
  // argument first and then returns SIA_ERR_WORKSPACE for a missing one, so
  // nothing touches the device and the status is the one that call documents.
  if (need == (size_t)-1 || need == 0 || need > sia::kNoAllocScratchBytes)
    return sia_index_select_attend(in, q_mla, q_dtype, heads, kv, seq, K, order, softmax_scale, idx_out, out, lse,
                                   nullptr, 0, stream);
  void* ws = nullptr;
  const hipError_t e = sia::scratch_on_current_device(&ws);
  if (e != hipSuccess) return sia::record_hip_error(e);
  return sia_index_select_attend(in, q_mla, q_dtype, heads, kv, seq, K, order, softmax_scale, idx_out, out, lse, ws,
                                 sia::kNoAllocScratchBytes, stream);
}

}  // extern "C"

// Host-only stand-ins for what the C ABI layer (sia_api.cpp) calls, so that it
// can be built and exercised under AddressSanitizer / UBSan without a GPU:
// the HIP runtime queries it makes, and the kernel launchers and size helpers
// of the kernel sources.  Launchers only count their calls; sizes follow the
// same shape as the real helpers (a per-row candidate list, split partials).
#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

#include "../../sparse_index_attention_amd/csrc/sia_internal.hpp"

int g_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace sia {
hipError_t launch_index_scores(const sia_indexer_in&, const SeqArgs&, float*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_topk(const float*, int64_t, const SeqArgs&, int, int, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_topk_pages(const float*, int64_t, const SeqArgs&, int, int32_t*, float*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quantize_q(const void*, int, int, int, bool, uint8_t*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_index_topk(const sia_indexer_in&, const SeqArgs&, int, int, int32_t*, float*, float*, int32_t*,
                             hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_sparse_mla(const void*, int, const sia_kv_in&, const SeqArgs&, const int32_t*, int, float, void*,
                             float*, int, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int index_topk_ranges(int max_visible) { return (max_visible + kIndexTopkRangeKeys - 1) / kIndexTopkRangeKeys; }
int64_t index_topk_ld(int max_visible, int K) { return ((int64_t)index_topk_ranges(max_visible) * K + 3) / 4 * 4; }
size_t topk_pages_ws_bytes(int T, int max_visible, int K) {
  return (size_t)T * ((size_t)(max_visible + 63) / 64 + (size_t)K / 64) * 8 + 256;
}
int mla_splits(int T, int K, int) { return T >= 256 ? 1 : (K + 255) / 256; }
size_t mla_workspace_bytes(int T, int K, int heads, int latent) {
  const int s = mla_splits(T, K, heads);
  return s <= 1 ? 0 : (size_t)T * s * heads * ((size_t)latent * 2 + 4) + 256;
}
}  // namespace sia

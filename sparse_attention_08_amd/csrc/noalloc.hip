// dsa_indexer_topk_noalloc: dsa_indexer_topk for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Its workspace is a file-scope device array instead
// of a caller buffer; the kernels are those of dsa_indexer_topk.
//
// In host code `scratch` names a host-side stand-in, not the device array: its
// device address is looked up once per device with hipGetSymbolAddress (each
// GPU holds its own copy, at its own address) and only that address is passed
// to kernels.  Nothing here calls hipMalloc, hipFree or any allocating routine.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsa.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // DSA_NOALLOC_SCRATCH_BYTES in dsa.h
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The scratch array's device address on the current device (looked up on the
// first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return DSA_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DSA_OK;
}

}  // namespace

extern "C" int dsa_indexer_topk_noalloc(const void* q, const void* k, const float* k_scale,
                                        const float* w, const int32_t* row_starts,
                                        const int32_t* row_ends, int64_t n_q, int64_t n_k,
                                        int32_t n_heads, int32_t head_dim, int32_t dtype,
                                        int32_t index_topk, int32_t* topk_idx, void* stream) {
  static_assert(DSA_NOALLOC_SCRATCH_BYTES == kScratchBytes, "header and library agree");
  const size_t need =
      dsa_indexer_topk_workspace_size(n_q, n_k, n_heads, head_dim, dtype, index_topk);
  if (need > kScratchBytes) return DSA_ERR_WORKSPACE;
  if (need == 0)
    return dsa_indexer_topk(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, head_dim,
                            dtype, index_topk, topk_idx, nullptr, 0, stream);
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != DSA_OK) return st;
  return dsa_indexer_topk(q, k, k_scale, w, row_starts, row_ends, n_q, n_k, n_heads, head_dim,
                          dtype, index_topk, topk_idx, ws, kScratchBytes, stream);
}

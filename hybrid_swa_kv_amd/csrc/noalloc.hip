// attn_decode_int8kv without a caller workspace: the split records go to a
// file-scope device array instead (for callers that cannot allocate device
// memory: code under graph capture, tight serving loops).
//
// The array is not addressable from host code by its name: its host-side symbol
// is a stand-in.  Its device address is looked up once per device, with that
// device current, by hipGetSymbolAddress, and only that address is handed to the
// kernels.  Each GPU holds its own copy for the life of the process.  Every call
// on a device shares that device's copy, so calls that overlap on one GPU (two
// streams, or two host threads) race on it; calls in stream order do not.  The
// decode writes every split record it later reads, so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hybrid_swa_kv.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = ATTN_DECODE_INT8KV_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of this device's `scratch` (looked up on first use).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HSK_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HSK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HSK_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return HSK_OK;
}

}  // namespace

extern "C" int attn_decode_int8kv_noalloc(const void* q, const int8_t* k_codes, const float* k_scales,
                                          const int8_t* v_codes, const float* v_scales, const void* k_hot,
                                          const void* v_hot, void* out, int B, int Hq, int Hkv, int D, int T8,
                                          int Th, float scale, void* stream) {
  // every argument error, then the size limit, before any HIP call
  if (int rc = hsk::int8_decode_validate(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, out, B, Hq, Hkv,
                                         D, T8, Th, scale))
    return rc;
  if (attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th) > kScratchBytes) return HSK_ERR_WORKSPACE;
  void* ws = nullptr;
  if (int rc = scratch_ptr(&ws)) return rc;
  return attn_decode_int8kv(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, out, B, Hq, Hkv, D, T8, Th,
                            scale, ws, kScratchBytes, stream);
}

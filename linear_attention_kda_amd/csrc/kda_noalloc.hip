// kda_fwd_noalloc: the forward pass with its workspace in a static device array
// instead of memory taken from the library's pool, for callers that cannot
// allocate (HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this translation unit's code object, which the runtime
// loads (and so reserves the array on a device) only when this file's symbol
// is first looked up on that device.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that
// address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, float scale, const void* initial_state,
                                      int initial_dtype, void* final_state, int final_dtype,
                                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                                      int64_t T, int32_t H, int32_t K, int32_t V, void* out,
                                      void* stream) {
  // argument errors first, exactly as kda_fwd reports them
  const kda_status st = kda_fwd_check(q, k, v, g, beta, scale, initial_state, initial_dtype,
                                      final_state, final_dtype, cu_seqlens, num_seqs, B, T, H, K,
                                      V, out);
  if (st != KDA_OK) return st;
  kda::ExtWorkspace ext{nullptr, KDA_NOALLOC_SCRATCH_BYTES};
  const hipError_t err = scratch_address(&ext.ptr);
  if (err != hipSuccess) {
    char text[160];
    snprintf(text, sizeof text, "static scratch lookup (hipGetSymbolAddress): %s",
             hipGetErrorString(err));
    return kda::record_failure(KDA_ERR_HIP, text);
  }
  return kda::fwd_impl(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state,
                       final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out, stream, false, &ext);
}

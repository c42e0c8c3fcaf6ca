// Library-owned split-KV scratch for the decode entry point that allocates
// nothing (fa_decode_paged_noalloc): code under HIP graph capture, serving
// loops and harnesses that forbid hipMalloc cannot hand the library a
// workspace, so the partial outputs and log-sum-exps of a key-split decode go
// to this file-scope device array instead. Each GPU the library runs on holds
// its own copy, at its own address, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (with that device current) by
// hipGetSymbolAddress and cached, and only that address is ever passed to a
// kernel. Every call on one GPU shares the array and finds the previous
// call's contents in it; the decode kernels write every partial row and lse
// they read back, so nothing has to start at zero. Calls that overlap on one
// GPU (different streams, no ordering) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fa_kernels.h"

namespace fa {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t device_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fa

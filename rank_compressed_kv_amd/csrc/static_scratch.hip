// Library-owned device scratch for palu_decode_attn_noalloc, the decode entry
// point for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch is one file-scope device array per GPU (the loader places a copy
// on every device the library runs on; each copy lives until the process
// ends). Host code never uses the array's name as an address: the name is a
// host-side stand-in. The device address of each GPU's copy is looked up once
// with hipGetSymbolAddress, with that device current, and kept per device;
// kernels receive that address as their workspace argument. Every call on a
// GPU shares that GPU's copy, so calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "palu_internal.h"

namespace palu {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[device].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[device].load(std::memory_order_relaxed);
    if (!p) {
      // the caller made `device` current
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[device].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace palu

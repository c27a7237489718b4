// noalloc.hip -- the device scratch behind mxfp4_quantize_noalloc, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The NVFP4 tensor-amax pass writes one 32-bit partial maximum per workgroup
// and the finalize reads them back; the no-allocation entry point keeps them
// in this file-scope array instead of a caller's workspace.  Every partial is
// written before it is read, so nothing needs clearing between calls.  Each
// device holds its own copy for the life of the process, shared by every
// call on that device: calls that overlap on one device race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mxfp4_internal.h"

namespace mxfp4 {

constexpr size_t kNoallocScratchBytes = (size_t)1 << 20;   // 262144 partials

static __device__ __align__(256) uint32_t scratch[kNoallocScratchBytes / sizeof(uint32_t)];

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of the current device's copy is looked up once per device
// (with that device current) and kept.
hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace mxfp4

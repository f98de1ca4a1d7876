// A library-owned device buffer for rr_decode_noalloc, the entry point for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from the code object's load until the
// process ends. In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is ever
// handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <atomic>

#include "rr_kernels.h"

namespace rr {

static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

hipError_t static_workspace(hipStream_t st, void** ptr) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the lookup needs the stream's device current; restore the caller's after
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);  // racing first calls store the same address
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace rr

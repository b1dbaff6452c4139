// Library-owned scratch for the sketch entry point that allocates nothing
// (logra_sketch_accumulate_noalloc, for callers that cannot allocate device
// memory: code under stream capture, tight loops, allocation-free harnesses).
//
// The scratch is one file-scope device array of kNoallocScratchBytes.  Each
// GPU the library runs on holds its own copy at its own address until the
// process ends.  In host code the array's name is only a host-side stand-in,
// never a device address.  The device address comes from
// hipGetSymbolAddress, called once per device with that device current, and
// is kept per device; kernels receive that pointer as their workspace.
// Every call on a GPU shares that GPU's array and finds the previous call's
// contents there (the sketch kernels overwrite everything they read before
// reading it).  Two calls that overlap on one GPU race on the array.
#include <mutex>

#include "internal.hpp"

namespace logra {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e;
  if (s != nullptr) {
    hipDevice_t sd;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return e;
    dev = (int)sd;
  } else {
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace logra

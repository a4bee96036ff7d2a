// The fixed device scratch behind dv_verify_rows_noalloc: the entry point for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc). The noise table that
// dv_verify_rows otherwise builds in a caller's workspace goes here instead.
//
// The array is a file-scope device variable, so each GPU the library runs on
// holds its own copy from the time the code object is loaded until the process
// ends. In host code its name is only a host-side stand-in, never a device
// address: the device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept, and only that
// address is handed to kernels. Every call on a device shares the one copy and
// overwrites it; calls that overlap on one device race.
#include <atomic>

#include "dv_internal.h"

static __device__ __align__(256) unsigned char scratch[DV_NOALLOC_SCRATCH_BYTES];

namespace dv {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void **ptr) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // first call on this device: resolve the symbol with the device current
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace dv

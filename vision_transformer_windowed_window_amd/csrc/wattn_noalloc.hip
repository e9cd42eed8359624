// wattn_noalloc.hip -- the library-held scratch of wattn_backward_noalloc (libwattn.so, gfx950).
//
// Callers that cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc) get the backward pass's scratch from this file-scope device
// array instead of a workspace argument.  Every GPU that the library runs on holds its own copy
// of the array, from the loading of the library's code object until the process ends.  The
// array's name is a host-side stand-in in host code, not a device address: its address on a
// device comes from hipGetSymbolAddress with that device current, once per device, and only
// that address is ever handed to a kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "wattn_noalloc.h"

namespace {

static __device__ __align__(256) unsigned char scratch[WATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` per device, filled on first use

}  // namespace

// Device address of the scratch array on the device that `stream` belongs to (the current
// device for the null stream).  The first call for a device makes that device current for the
// lookup and restores the caller's device afterwards.
hipError_t wattn_noalloc_scratch(hipStream_t stream, void** out) {
  *out = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

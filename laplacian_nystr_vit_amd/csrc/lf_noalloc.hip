// The device scratch array behind lf_attn_fwd_noalloc: the forward workspace for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array; every GPU the library runs on holds its own copy from the first launch
// on that device until the process ends. In host code its name is only a host-side stand-in, so the device
// address is looked up once per device with hipGetSymbolAddress (with that device current) and kept; launches,
// copies and fills use that address, never the array's name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lf_attn.h"
#include "lf_internal.h"

namespace lf {

namespace {

static __device__ __align__(256) unsigned char scratch[LF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t st, void** out) {
  *out = nullptr;
  hipDevice_t dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);  // the null stream is the current device's
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace lf

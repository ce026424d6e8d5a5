// The split-K scratch of pa_decode_noalloc: a fixed device array, so that the
// call never allocates (for callers that cannot, such as code under graph
// capture or serving loops that forbid allocation).
//
// The array is a __device__ variable: every GPU the library runs on holds its
// own copy, at its own address, from the moment the library's code is loaded
// on that GPU until the process ends.  In host code the name `scratch` is only
// a stand-in for the device symbol -- it is not a device address -- so the
// address of each GPU's copy is looked up once, with hipGetSymbolAddress on
// that GPU, and only that looked-up address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "pa.h"

static __device__ __align__(256) char scratch[PA_DECODE_NOALLOC_MAX_WORKSPACE];

namespace pa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU, once looked up

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    // The lookup runs with the stream's device current, so it returns that
    // GPU's copy of the array; the caller's current device is restored.
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace pa

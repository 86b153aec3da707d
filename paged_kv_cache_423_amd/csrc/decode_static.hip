// The decode's partition partials in a buffer the library owns, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): pkv_paged_attention_
// decode_static in api.cpp takes its workspace from here.
//
// `scratch` is one file-scope device array of PKV_STATIC_WORKSPACE_BYTES; each
// GPU the library runs on holds its own copy at its own address until the
// process ends.  In host code its name is only a host-side stand-in, so the
// device address is looked up once per device, with that device current,
// through hipGetSymbolAddress, and only that address is ever handed to a
// kernel.  Every call on one GPU shares that GPU's copy; the decode writes
// every partial it reads within the same call, so nothing needs clearing,
// and calls that overlap on one GPU (different streams at once) race.

#include <mutex>

#include "pagedkv.h"
#include "decode_static.h"

static __device__ __align__(256) unsigned char scratch[PKV_STATIC_WORKSPACE_BYTES];

namespace pkv {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];    // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t static_workspace(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace pkv

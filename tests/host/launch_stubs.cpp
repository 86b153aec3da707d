// Host-only stand-ins for libpagedkv's kernel launchers, linked instead of
// the HIP kernel sources into the sanitizer build of the C ABI's host code
// (abi_harness.cpp).  Each records that it was reached and launches nothing.

#include "checks.h"
#include "decode_static.h"
#include "kernels.h"

int pkv_stub_launches = 0;
int pkv_stub_static_lookups = 0;
alignas(256) static unsigned char pkv_stub_static_ws[1024];

namespace pkv {

static hipError_t reached() {
  ++pkv_stub_launches;
  return hipSuccess;
}

hipError_t launch_paged_decode_partitions(const DecodeArgs&, hipStream_t) { return reached(); }
hipError_t launch_paged_decode_merge(const DecodeArgs&, hipStream_t) { return reached(); }
hipError_t launch_paged_decode(const DecodeArgs&, hipStream_t) { return reached(); }
hipError_t static_workspace(void** ptr) {
  ++pkv_stub_static_lookups;
  *ptr = pkv_stub_static_ws;
  return hipSuccess;
}
hipError_t launch_paged_prefill(const PrefillArgs&, hipStream_t) { return reached(); }
hipError_t launch_reshape_and_cache(const void*, const void*, void*, void*, const int32_t*, int, int, int, int, int,
                                    int, int, float, float, const float*, const float*, hipStream_t) {
  return reached();
}
hipError_t launch_copy_blocks(void*, void*, const int32_t*, int, int, size_t, hipStream_t) { return reached(); }
hipError_t launch_swap_blocks(void*, void*, const void*, const void*, const int32_t*, int, int, int, size_t,
                              hipStream_t) {
  return reached();
}
hipError_t launch_gather_kv(void*, void*, const int32_t*, const void*, const void*, const int32_t*, const int32_t*, int,
                            int, int, int, int, int, int, hipStream_t) {
  return reached();
}
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) { return reached(); }
hipError_t launch_check_step_inputs(const int32_t*, const int32_t*, int, int, const int32_t*, int, const int32_t*, int,
                                    int, int, int, uint32_t*, hipStream_t) {
  return reached();
}

}  // namespace pkv

// The static decode workspace of pkv_paged_attention_decode_static
// (internal; see decode_static.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

// Device address of this device's copy of the static decode workspace
// (PKV_STATIC_WORKSPACE_BYTES), looked up on the first call on each device
// with that device current.
hipError_t static_workspace(void** ptr);

}  // namespace pkv

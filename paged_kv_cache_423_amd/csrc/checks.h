// Host-side launcher of the step-input check (internal; the public C ABI is
// include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Layout of the check's workspace, in 32-bit words from its start: word 0
// the violation mask, then the slot bitmap (NB * BS bits), the copy-source
// and copy-destination bitmaps (NB bits each) and one map count per block,
// each section starting on a 256-byte boundary.
struct CheckLayout {
  size_t slot_bm, src_bm, dst_bm, counts, words;
};
inline CheckLayout check_layout(int NB, int BS) {
  auto up = [](size_t x) { return (x + 63) / 64 * 64; };   // 256-byte sections
  CheckLayout L;
  L.slot_bm = 64;                                           // word 0: the mask; the rest of the first 256 B unused
  L.src_bm = L.slot_bm + up(((size_t)NB * BS + 31) / 32);
  L.dst_bm = L.src_bm + up(((size_t)NB + 31) / 32);
  L.counts = L.dst_bm + up(((size_t)NB + 31) / 32);
  L.words = L.counts + up((size_t)NB);
  return L;
}

// Clears the workspace and runs the two check passes; the mask is in word 0
// when they finish.  tables / lens may be null when S == 0, slots when
// T == 0, pairs when N == 0; append requires T == S.
hipError_t launch_check_step_inputs(const int32_t* block_tables, const int32_t* context_lens, int S, int MB,
                                    const int32_t* slot_mapping, int T, const int32_t* pairs, int N, int BS, int NB,
                                    int append, uint32_t* workspace, hipStream_t stream);

}  // namespace pkv

// Device-side validation of one step's index inputs: the block tables and
// context lengths ("vLLM-v0.17.1技术解析" §2.2, "在A10G上榨干LLaMA-7B" §2.1),
// the int32 slot mapping of the new tokens (the l189.com article on KV cache
// and slot mapping, §2.2) and the copy-on-write block pairs ("在A10G上榨干
// LLaMA-7B" §2.2).  The other kernels never fault on such inputs (they clamp
// lengths and block ids and skip slots past the pool), but their results are
// then unspecified; this pass says which condition a step breaks.
//
// Three launches over a caller-provided workspace of 32-bit words:
//   1. clear the workspace (a fill kernel);
//   2. one thread per used-or-not table entry, per slot and per copy pair:
//      range checks; each used entry adds 1 to its block's map count; each
//      slot sets its bit in a slot bitmap (atomic OR: a bit already set is a
//      duplicate); each pair sets its source bit and its destination bit (a
//      destination bit already set is a repeat);
//   3. one thread per slot and per pair, after every map count and bitmap is
//      complete: a written slot in a block mapped more than once, a
//      destination that is also a source, and, for the appending decode, a
//      slot that is not the one of its sequence's position n - 1.
// Every violation ORs its bit into word 0.  Only vector atomics are used.

#include <algorithm>

#include "checks.h"

namespace pkv {

namespace {

constexpr uint32_t kContextLen = 1u << 0;
constexpr uint32_t kBlockId = 1u << 1;
constexpr uint32_t kSlotRange = 1u << 2;
constexpr uint32_t kSlotDup = 1u << 3;
constexpr uint32_t kPairRange = 1u << 4;
constexpr uint32_t kPairOverlap = 1u << 5;
constexpr uint32_t kAppendSlot = 1u << 6;
constexpr uint32_t kSharedWrite = 1u << 7;

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_clear_kernel(uint32_t* __restrict__ ws, size_t words) {
  for (size_t i = (size_t)blockIdx.x * kCheckThreads + threadIdx.x; i < words; i += (size_t)gridDim.x * kCheckThreads)
    ws[i] = 0u;
}

__global__ __launch_bounds__(kCheckThreads) void check_pass1_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, int S, int MB,
    const int32_t* __restrict__ slots, int T, const int32_t* __restrict__ pairs, int N, int BS, int NB,
    uint32_t* __restrict__ ws, CheckLayout L) {
  const size_t i = (size_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const size_t E = (size_t)S * MB;
  uint32_t bad = 0;
  if (i < E) {
    const int s = (int)(i / MB), j = (int)(i % MB);
    const int64_t cap = (int64_t)MB * BS;
    const int raw = lens[s];
    if (j == 0 && (raw < 0 || raw > cap)) bad |= kContextLen;
    const int64_t n = raw < 0 ? 0 : (raw > cap ? cap : raw);
    if (j < (n + BS - 1) / BS) {
      const int b = tables[i];
      if (b < 0 || b >= NB) bad |= kBlockId;
      else atomicAdd(ws + L.counts + b, 1u);
    }
  } else if (i < E + (size_t)T) {
    const int slot = slots[i - E];
    if (slot >= 0) {
      if ((int64_t)slot >= (int64_t)NB * BS) {
        bad |= kSlotRange;
      } else {
        const uint32_t bit = 1u << (slot & 31);
        if (atomicOr(ws + L.slot_bm + (slot >> 5), bit) & bit) bad |= kSlotDup;
      }
    }
  } else if (i < E + (size_t)T + (size_t)N) {
    const size_t k = i - E - T;
    const int src = pairs[2 * k], dst = pairs[2 * k + 1];
    if (src < 0 || src >= NB || dst < 0 || dst >= NB) {
      bad |= kPairRange;
    } else {
      atomicOr(ws + L.src_bm + (src >> 5), 1u << (src & 31));
      const uint32_t bit = 1u << (dst & 31);
      if (atomicOr(ws + L.dst_bm + (dst >> 5), bit) & bit) bad |= kPairOverlap;
    }
  }
  if (bad) atomicOr(ws, bad);
}

__global__ __launch_bounds__(kCheckThreads) void check_pass2_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, int MB,
    const int32_t* __restrict__ slots, int T, const int32_t* __restrict__ pairs, int N, int BS, int NB,
    int append, uint32_t* __restrict__ ws, CheckLayout L) {
  const size_t i = (size_t)blockIdx.x * kCheckThreads + threadIdx.x;
  uint32_t bad = 0;
  if (i < (size_t)T) {
    const int slot = slots[i];
    if (slot >= 0 && (int64_t)slot < (int64_t)NB * BS && ws[L.counts + slot / BS] > 1u) bad |= kSharedWrite;
    if (append && slot >= 0) {               // one token per sequence: token i is sequence i's
      const int64_t cap = (int64_t)MB * BS;
      const int raw = lens[i];
      const int64_t n = raw < 0 ? 0 : (raw > cap ? cap : raw);
      if (n == 0) {
        bad |= kAppendSlot;
      } else {
        const int64_t t = n - 1;
        const int64_t want = (int64_t)tables[i * (size_t)MB + t / BS] * BS + t % BS;
        if ((int64_t)slot != want) bad |= kAppendSlot;
      }
    }
  }
  if (i < (size_t)N) {
    const int src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src >= 0 && src < NB && dst >= 0 && dst < NB && (ws[L.src_bm + (dst >> 5)] >> (dst & 31) & 1u))
      bad |= kPairOverlap;
  }
  if (bad) atomicOr(ws, bad);
}

unsigned grid_for(size_t items) { return (unsigned)((items + kCheckThreads - 1) / kCheckThreads); }

}  // namespace

hipError_t launch_check_step_inputs(const int32_t* tables, const int32_t* lens, int S, int MB, const int32_t* slots,
                                    int T, const int32_t* pairs, int N, int BS, int NB, int append, uint32_t* ws,
                                    hipStream_t stream) {
  const CheckLayout L = check_layout(NB, BS);
  hipLaunchKernelGGL(check_clear_kernel, dim3(std::min<size_t>(grid_for(L.words), 1024)), dim3(kCheckThreads), 0,
                     stream, ws, L.words);
  const size_t items1 = (size_t)S * MB + (size_t)T + (size_t)N;
  if (items1 > 0)
    hipLaunchKernelGGL(check_pass1_kernel, dim3(grid_for(items1)), dim3(kCheckThreads), 0, stream, tables, lens, S,
                       MB, slots, T, pairs, N, BS, NB, ws, L);
  const size_t items2 = std::max<size_t>((size_t)T, (size_t)N);
  if (items2 > 0)
    hipLaunchKernelGGL(check_pass2_kernel, dim3(grid_for(items2)), dim3(kCheckThreads), 0, stream, tables, lens, MB,
                       slots, T, pairs, N, BS, NB, append, ws, L);
  return hipGetLastError();
}

}  // namespace pkv

// Host-side launchers of the libpagedkv kernels (internal; the public C ABI is
// include/pagedkv.h).  Every launcher enqueues on the given stream and
// returns hipGetLastError() of its launches; arguments are validated by the
// caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int S, H, D, BS, MB, NB;
  int q_fmt, c_fmt;
  float q_mult;    // scale * log2(e), times k_scale for 8-bit pools with one scale per pool
  float out_mult;  // v_scale for 8-bit pools with one scale per pool, else 1
  // 8-bit pools with one scale per head: fp32 [H] on the device, each
  // multiplying q_mult (k_scales) and out_mult (v_scales) for its head;
  // null otherwise
  const float* k_scales;
  const float* v_scales;
  int group_size;  // > 1: groups of this many consecutive sequences share the
                   // loads of blocks they all map (16-bit and f32 pools)
  float* ws_ml;    // [S][H][max_parts][2] partition (max, sum)
  float* ws_acc;   // [S][H][max_parts][D] partition weighted V
  // set when the decode also writes the step's new tokens (one per
  // sequence, [S][H][D] in the q format) at slot_mapping; null otherwise
  const void* new_k;
  const void* new_v;
  const int32_t* slot_mapping;
  float k_scale, v_scale;  // divisors of the 8-bit pools' write
};

// Tokens per context partition of the decode kernel (the workspace size
// depends on it): 128 physical blocks of 16 tokens, 64 of 32.  Contexts up
// to this length need no merge phase.
constexpr int kPartTokens = 2048;

// Largest group of sequences the grouped decode reduces together.
constexpr int kMaxGroup = 8;
constexpr int part_blocks(int BS) { return kPartTokens / BS; }

// The two phases of the decode: the partition kernel (writes the output of
// sequences that fit one partition, partials otherwise) and the merge of the
// partials.  launch_paged_decode runs both.
hipError_t launch_paged_decode_partitions(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_paged_decode_merge(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  int S, Tq, max_q_len, H, D, BS, MB, NB;
  int fmt;         // q and output format (F16 or BF16)
  int c_fmt;       // pool format: fmt, E4M3 or I8
  float s_mult;    // scale * log2(e) (* k_scale for 8-bit pools with one scale per pool)
  float out_mult;  // v_scale for 8-bit pools with one scale per pool, else 1
  float k_scale, v_scale;   // 8-bit pools: the scales the cache write divides by
  const float* k_scales;    // 8-bit pools with one scale per head: fp32 [H] (else null),
  const float* v_scales;    // multiplying s_mult / out_mult and dividing in the cache write
  // set when the kernel also stores the new tokens' K/V ([Tq][H][D]) at
  // slot_mapping; null otherwise
  const void* new_k;
  const void* new_v;
  const int32_t* slot_mapping;
};

// Multi-query (prompt) attention over the paged cache, causal by position.
hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream);

// k_scales / v_scales: one scale per head (fp32 [H] on the device) in place
// of k_scale / v_scale, or null.
hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int T, int H, int D, int BS, int NB,
                                    int src_fmt, int c_fmt, float k_scale, float v_scale,
                                    const float* k_scales, const float* v_scales, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int N, int NB,
                              size_t block_bytes, hipStream_t stream);

// Block copies from one pool pair to another; any of the pointers may be a
// device address of pinned host memory.
hipError_t launch_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int N, int NB_src, int NB_dst, size_t block_bytes,
                              hipStream_t stream);

hipError_t launch_gather_kv(void* k_out, void* v_out, const int32_t* cu_lens, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int S, int H, int D, int BS, int MB,
                            int NB, int c_fmt, hipStream_t stream);

// Read-only stream over a device buffer (bandwidth probe); bytes is a
// multiple of 16.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace pkv

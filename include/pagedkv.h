/*
 * pagedkv.h: C ABI of libpagedkv.so, paged-attention decode for AMD gfx950.
 *
 * Method (pages cited by title and section):
 *   [P1] "vLLM-v0.17.1技术解析：PagedAttention内存管理与显存优化技巧"
 *   [P2] "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战"
 *   [P3] the l189.com article on KV cache, PagedAttention, slot mapping and
 *        CUDA graphs (www.l189.com/news/180929)
 *
 * The KV cache is split into fixed-size physical blocks that are allocated
 * and freed one at a time ([P1] §2.2, [P3] §2.1).  A sequence's tokens fill
 * logical blocks in order; a per-sequence block table maps each logical
 * block to a physical block anywhere in the pool ([P2] §2.1).  New tokens'
 * K/V are written to the slots an int32 slot mapping names ([P3] §2.2).
 * Sequences with a common prefix map the same physical blocks and copy a
 * block before writing into it while it is still shared ([P2] §2.2).
 *
 * Layouts (all row-major, element type given by a pkv_dtype):
 *   k_cache, v_cache  [NB][H][BS][D]   one pool each for K and V; one
 *                                      (block, head) tile is BS rows of D
 *                                      contiguous elements.
 *   q, out            [S][H][D]        one query token per head per sequence.
 *   key, value        [T][H][D]        the T new tokens' K and V.
 *   slot_mapping      int32 [T]        slot = block * BS + offset; a negative
 *                                      slot skips the token (padding).
 *   block_tables      int32 [S][MB]    physical block of logical block j of
 *                                      sequence s; entries at j >= ceil(n_s/BS)
 *                                      are never read.
 *   context_lens      int32 [S]        n_s tokens of sequence s are attended
 *                                      (the token appended this step included),
 *                                      0 <= n_s <= MB * BS.
 * Cache element types: PKV_F32, PKV_F16, PKV_BF16 hold the value itself;
 * PKV_FP8_E4M3 holds OCP E4M3FN bytes of value / scale with one fp32 scale per
 * pool (k_scale for K, v_scale for V): the cached value is byte * scale.
 * PKV_INT8 holds two's-complement bytes of value / scale in the same way
 * ([P1] §3.3 lists INT8 beside FP8 as an 8-bit format; [P3] §4 speaks of a
 * quantised cache in FP8 "and similar formats"): cached value = byte * scale.
 * An 8-bit pool may instead carry one fp32 scale per head: the *_head_scales
 * entry points take k_scales / v_scales, fp32 [H] arrays in device memory
 * (4-byte aligned, finite and > 0; their contents are read on the device and
 * not checked), in place of k_scale / v_scale, and head h's rows are stored
 * as value / k_scales[h] and read as byte * k_scales[h] (likewise V).  The
 * pages do not say how finely a scale applies; one scale per pool is the
 * case of equal per-head scales, and gives the same bits.  For F32, F16 and
 * BF16 pools the arrays are ignored (and may be NULL).
 *
 * Conventions for every call:
 *   - Every pointer is a device pointer owned by the caller (pkv_swap_blocks
 *     also takes pinned host memory).  Apart from the decode-graph objects,
 *     which the caller creates and destroys (pkv_decode_graph_*), and the
 *     static decode workspace each GPU holds for
 *     pkv_paged_attention_decode_static, the library allocates nothing and
 *     keeps no state between calls; calls are thread-safe (overlapping
 *     pkv_paged_attention_decode_static calls on one GPU race on that
 *     workspace).
 *   - Work is enqueued on `stream` (NULL = the null stream) and the call
 *     returns without synchronising (except pkv_check_step_inputs, which
 *     reads its result back).
 *   - Host-side checks, done before anything is enqueued:
 *       PKV_ERR_INVALID_ARG  null pointer, non-positive size, negative count,
 *                            non-finite or non-positive scale.
 *       PKV_ERR_UNSUPPORTED  a shape or dtype combination outside the
 *                            supported set: D in {64, 80, 96, 128, 256},
 *                            BS in {16, 32},
 *                            (q, cache) in {(F32,F32), (F16,F16), (BF16,BF16),
 *                            (F16,FP8_E4M3), (BF16,FP8_E4M3), (F16,INT8),
 *                            (BF16,INT8)}; for the cache write the source
 *                            dtype is the q dtype.  Grid limits: S at most
 *                            65535 (decode, prompt attention, gather), H at
 *                            most 65535 (decode, prompt attention), tables of at most
 *                            65535 partitions of 2048 tokens for the decode,
 *                            and prompts of at most 65535 * 128 new tokens.
 *       PKV_ERR_WORKSPACE    workspace smaller than pkv_decode_workspace_bytes.
 *       PKV_ERR_HIP          the launch failed (hipGetLastError).
 *   - Device-side contents are not validated by the compute calls, but no
 *     kernel access leaves the buffers because of them: a context length
 *     outside [0, MB*BS] is clamped into it, a block id outside [0, NB) reads
 *     block 0 instead, a slot past the pool and a copy pair naming a block
 *     outside it are skipped.  Such inputs, two tokens naming one slot, and
 *     copy pairs whose destination repeats or is also a source give
 *     unspecified results.  pkv_check_step_inputs (the one call that
 *     synchronises) checks them on request and returns
 *     PKV_ERR_DEVICE_CHECK with a mask of the conditions broken.
 *   - No C++ exception crosses this interface.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,
  PKV_ERR_UNSUPPORTED = 2,
  PKV_ERR_WORKSPACE = 3,
  PKV_ERR_HIP = 4,
  PKV_ERR_DEVICE_CHECK = 5,  /* pkv_check_step_inputs found a violation */
  PKV_STATUS_MAX_ENUM = 0x7FFFFFFF   /* not a status: widens the type so that any
                                        non-negative int is a valid value in C++ */
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3,
  PKV_INT8 = 4,
  PKV_DTYPE_MAX_ENUM = 0x7FFFFFFF    /* not a dtype: widens the type so that an
                                        unknown non-negative code is refused, not
                                        undefined, in C++ */
} pkv_dtype;

/* Short English name of a status code (static storage, never NULL). */
const char* pkv_status_string(pkv_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int pkv_version(void);

/*
 * Write T new tokens' K and V into their cache slots ([P3] §2.2; [P2] §2.1,
 * where a generated token's K/V is stored in the block its sequence maps).
 * For token i with slot = slot_mapping[i] >= 0 and every head h:
 *   k_cache[slot / BS][h][slot % BS][:] = conv(key[i][h][:]), likewise v.
 * conv copies the bits when src_dtype == cache_dtype.  Into PKV_FP8_E4M3 it
 * computes the IEEE fp32 quotient x / k_scale (v_scale for V), rounded to
 * nearest even, and encodes it with round-to-nearest-even, saturating to
 * +-448 (infinities included); NaN becomes 0x7F.  Into PKV_INT8 the same
 * quotient is rounded to the nearest integer (ties to even) and saturated to
 * [-127, 127]; NaN becomes 0.
 *   key, value     [T][H][D] src_dtype.
 *   k_cache, v_cache [NB][H][BS][D] cache_dtype, updated in place.
 *   slot_mapping   int32 [T] on the device.
 * T = 0 is a no-op that returns PKV_OK.
 */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int32_t T, int32_t H, int32_t D,
                                 int32_t BS, int32_t NB, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                 float k_scale, float v_scale, hipStream_t stream);

/* pkv_reshape_and_cache with one scale per head of each 8-bit pool:
 * k_scales / v_scales are fp32 [H] on the device (NULL for an 8-bit pool is
 * PKV_ERR_INVALID_ARG).  Everything else as for pkv_reshape_and_cache. */
pkv_status pkv_reshape_and_cache_head_scales(const void* key, const void* value, void* k_cache, void* v_cache,
                                             const int32_t* slot_mapping, int32_t T, int32_t H, int32_t D,
                                             int32_t BS, int32_t NB, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                             const float* k_scales, const float* v_scales, hipStream_t stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for this shape
 * (0 when every context fits one partition of 2048 tokens, i.e. when
 * MB * BS <= 2048).  The contents need no
 * initialisation and are not read after the call's kernels finish.
 * Returns 0 for non-positive sizes.
 */
size_t pkv_decode_workspace_bytes(int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB);

/*
 * Single-query paged-attention decode ([P1] §2.2, [P2] §2.1): for every
 * sequence s and head h,
 *   z_t = scale * q[s][h] . K_s[t]          for t < n_s
 *   out[s][h] = sum_t softmax(z)_t * V_s[t]
 * where K_s[t] = k_cache[block_tables[s][t / BS]][h][t % BS] (times k_scale
 * for the 8-bit formats), likewise V_s.  n_s = 0 gives zeros.  Results do not depend on
 * where the blocks sit in the pool: the order of arithmetic depends only on
 * logical token positions, so two placements of the same tokens give
 * bitwise-equal outputs.
 *   out           [S][H][D] q_dtype (written).
 *   q             [S][H][D] q_dtype.
 *   k_cache, v_cache [NB][H][BS][D] cache_dtype.
 *   block_tables  int32 [S][MB];  context_lens int32 [S].
 *   scale         softmax scale, finite and > 0 (typically 1/sqrt(D)).
 *   k_scale, v_scale  fp8 / int8 pool scales, finite and > 0 (ignored otherwise).
 *   workspace     device scratch of at least
 *                 pkv_decode_workspace_bytes(S, H, D, BS, MB) bytes (may be
 *                 NULL when that is 0).
 * S = 0 is a no-op that returns PKV_OK.
 */
pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t S, int32_t H, int32_t D,
                                      int32_t BS, int32_t MB, int32_t NB, float scale,
                                      pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                                      float v_scale, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * The decode's two phases, for callers that want to time, overlap or
 * separately schedule them.  pkv_paged_attention_decode_partitions followed
 * by pkv_paged_attention_decode_merge, on one stream with the same
 * arguments, gives exactly the result of pkv_paged_attention_decode.
 *
 * _partitions: splits each context into partitions of 2048 tokens (128
 * physical blocks of 16 tokens, 64 of 32) and reduces each partition to (running max, sum of
 * exponentials, exponential-weighted sum of V), the online form of the
 * softmax; a sequence that fits one partition gets its output directly.
 * Arguments and checks as for pkv_paged_attention_decode.
 *
 * _merge: combines the partitions of every sequence longer than one
 * partition and writes its output.  It reads context_lens and the workspace
 * the partition phase wrote; the arguments carry the same meaning as above
 * (q_dtype is the output format, v_scale is used for fp8 pools).  It
 * enqueues nothing when the workspace size is 0.
 */
pkv_status pkv_paged_attention_decode_partitions(
    void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

pkv_status pkv_paged_attention_decode_merge(void* out, const int32_t* context_lens, int32_t S,
                                            int32_t H, int32_t D, int32_t BS, int32_t MB,
                                            pkv_dtype q_dtype, pkv_dtype cache_dtype, float v_scale,
                                            const void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/*
 * The decode of pkv_paged_attention_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels with the same results,
 * bit for bit, but the partition partials go to a static device buffer of
 * PKV_STATIC_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * until the process ends, instead of a caller workspace.  The call allocates
 * nothing.  The first call on a device looks the buffer's address up (with
 * that device current); later calls reuse it.
 *   Arguments as for pkv_paged_attention_decode, without the workspace.
 *   PKV_ERR_WORKSPACE  pkv_decode_workspace_bytes(S, H, D, BS, MB) exceeds
 *                      PKV_STATIC_WORKSPACE_BYTES (nothing is enqueued).
 *   PKV_ERR_HIP        the buffer's address could not be looked up, or the
 *                      launch failed.
 * Every call on one GPU shares that GPU's buffer, which keeps the last call's
 * partials: calls that overlap on one GPU (on different streams, or from
 * different threads, without ordering between them) race and give
 * unspecified results.  Calls ordered on one stream are safe.
 */
#define PKV_STATIC_WORKSPACE_BYTES ((size_t)16 << 20)

pkv_status pkv_paged_attention_decode_static(void* out, const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* block_tables,
                                             const int32_t* context_lens, int32_t S, int32_t H, int32_t D,
                                             int32_t BS, int32_t MB, int32_t NB, float scale,
                                             pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                                             float v_scale, hipStream_t stream);

/*
 * A decode step's cache write and attention in one pass: the token each
 * sequence generated is stored in the block its table maps, then attended
 * together with the rest of the context ([P2] §2.1: the new token's K/V are
 * stored, then used; [P3] §2.2: its slot comes from the slot mapping).
 * Equivalent, bit for bit in out and in both pools, to
 *   pkv_reshape_and_cache(key, value, ..., slot_mapping, T = S, ...)
 *   pkv_paged_attention_decode(out, q, ...)
 * For F32/F16/BF16 pools without a separate write kernel: the wave that reads
 * sequence s's last block uses the new row in place of what it loads for
 * position n_s - 1 and stores it into the pools.  For 8-bit pools the
 * cache-write kernel runs first (quantising inside the decode kernel would
 * cost it registers and occupancy).
 *   key, value    [S][H][D] q_dtype: one new token per sequence.
 *   slot_mapping  int32 [S]: the slot of that token, which must be the slot
 *                 of position context_lens[s] - 1 of sequence s (or negative
 *                 to skip the write, e.g. for a padding sequence with
 *                 n_s = 0).  That slot must not be read by another sequence
 *                 of the call, which copy-on-write of shared blocks ensures.
 *                 Otherwise the pools still receive the write, but the
 *                 output is unspecified (for F32/F16/BF16 pools the decode
 *                 takes the new row as position n_s - 1 either way; other
 *                 sequences reading the slot race with the write).
 * Other arguments, checks and the workspace as for
 * pkv_paged_attention_decode and pkv_reshape_and_cache; key and value must be
 * 16-byte aligned.  S = 0 is a no-op that returns PKV_OK.
 *
 * _append_partitions is its first phase; pkv_paged_attention_decode_merge
 * with the same arguments completes it, as for the decode's two phases.
 */
pkv_status pkv_paged_attention_decode_append(void* out, const void* q, const void* key, const void* value,
                                             void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                             const int32_t* block_tables, const int32_t* context_lens,
                                             int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB,
                                             int32_t NB, float scale, pkv_dtype q_dtype,
                                             pkv_dtype cache_dtype, float k_scale, float v_scale,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream);

pkv_status pkv_paged_attention_decode_append_partitions(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S,
    int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
    pkv_dtype cache_dtype, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/*
 * The decode for sequences that share blocks ([P2] §2.2: requests forked from
 * one prompt map the same physical blocks for it, which is stored once):
 * pkv_paged_attention_decode's result, bit for bit, with the reads of shared
 * blocks shared.  The sequences are taken in groups of group_size
 * consecutive ones (the last group may be smaller), and a group of more than
 * four runs as near-equal chunks of at most four; within a chunk, a logical
 * block that every sequence maps to the same physical block, before any
 * sequence's last block, is read from memory once and reduced into every
 * sequence's softmax state.  Every other block is read for its sequence
 * alone, so any tables are valid; sharing only saves reads.  Callers order
 * their batch so that sequences forked from one prompt are adjacent.
 *   group_size    1 .. 8 (1: the per-sequence decode).
 *   key, value, slot_mapping  all NULL, or all given for the appending step
 *                 (as in pkv_paged_attention_decode_append, whose result it
 *                 then gives: the grouped kernel stores each sequence's new
 *                 token and reads it in place of position n - 1).
 *   cache_dtype   PKV_F32, PKV_F16 or PKV_BF16, equal to q_dtype (8-bit pools
 *                 are PKV_ERR_UNSUPPORTED).
 * Other arguments, checks and the workspace as for pkv_paged_attention_decode.
 * _partitions is its first phase; pkv_paged_attention_decode_merge with the
 * same arguments completes it.
 */
pkv_status pkv_paged_attention_decode_grouped(void* out, const void* q, const void* key, const void* value,
                                              void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                              const int32_t* block_tables, const int32_t* context_lens, int32_t S,
                                              int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale,
                                              pkv_dtype q_dtype, pkv_dtype cache_dtype, int32_t group_size,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream);

pkv_status pkv_paged_attention_decode_grouped_partitions(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
    int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    int32_t group_size, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The decode's entry points with one scale per head of each 8-bit pool
 * (see the cache element types above): the same kernels, checks, workspace
 * and results as pkv_paged_attention_decode, _partitions, _merge, _append
 * and _append_partitions, with the device arrays k_scales / v_scales (fp32
 * [H]; NULL for an 8-bit pool is PKV_ERR_INVALID_ARG; _merge reads only
 * v_scales) in place of k_scale / v_scale.  The kernels multiply the q
 * scale by k_scales[h] and the output by v_scales[h], exactly as they do
 * with the pool's one scale.
 */
pkv_status pkv_paged_attention_decode_head_scales(void* out, const void* q, const void* k_cache,
                                                  const void* v_cache, const int32_t* block_tables,
                                                  const int32_t* context_lens, int32_t S, int32_t H, int32_t D,
                                                  int32_t BS, int32_t MB, int32_t NB, float scale,
                                                  pkv_dtype q_dtype, pkv_dtype cache_dtype, const float* k_scales,
                                                  const float* v_scales, void* workspace, size_t workspace_bytes,
                                                  hipStream_t stream);

pkv_status pkv_paged_attention_decode_partitions_head_scales(
    void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, const float* k_scales, const float* v_scales,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

pkv_status pkv_paged_attention_decode_merge_head_scales(void* out, const int32_t* context_lens, int32_t S,
                                                        int32_t H, int32_t D, int32_t BS, int32_t MB,
                                                        pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                                        const float* v_scales, const void* workspace,
                                                        size_t workspace_bytes, hipStream_t stream);

pkv_status pkv_paged_attention_decode_append_head_scales(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
    int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    const float* k_scales, const float* v_scales, void* workspace, size_t workspace_bytes, hipStream_t stream);

pkv_status pkv_paged_attention_decode_append_partitions_head_scales(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
    int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    const float* k_scales, const float* v_scales, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Multi-query (prompt) attention over the paged cache ([P2] §2.1 step 1: a
 * prompt's K/V are stored in the blocks allocated for it, then used; [P2]
 * §2.2: a prompt prefix shared by several requests is stored once, so a
 * request whose prefix is cached computes only its own new tokens; [P1]
 * §3.2: attention as one fused kernel).  Sequence s holds n_s =
 * context_lens[s] tokens in the cache, the last q_s = cu_q_lens[s + 1] -
 * cu_q_lens[s] of them new (their K/V already written, e.g. by
 * pkv_reshape_and_cache).  New token i sits at position n_s - q_s + i and
 * attends to positions 0 .. n_s - q_s + i:
 *   z_t = scale * q[cu_q_lens[s] + i] . K_s[t]
 *   out[cu_q_lens[s] + i] = sum_t softmax(z)_t * V_s[t]
 * with K_s, V_s read through the block table as for the decode (times
 * k_scale / v_scale for 8-bit pools).  One new token per sequence gives the
 * decode's result.  The products run on the matrix cores with fp32
 * accumulation in the q format; 8-bit pool values are converted to it
 * exactly (every E4M3 and INT8 value is an fp16 and a bf16 value), and the
 * scales are applied to the scores and to the output.  The softmax weights
 * are rounded to the q format before they multiply V.
 *   out           [Tq][H][D] q_dtype (written, rows of the new tokens).
 *   q             [Tq][H][D] q_dtype, the new tokens' queries, packed by sequence.
 *   k_cache, v_cache [NB][H][BS][D] cache_dtype.
 *   block_tables  int32 [S][MB];  context_lens int32 [S] (new tokens included).
 *   cu_q_lens     int32 [S + 1] on the device: cu_q_lens[0] = 0, non-decreasing,
 *                 cu_q_lens[S] = Tq, q_s <= min(n_s, max_q_len).
 *   max_q_len     the largest q_s (sets the grid).
 *   scale         softmax scale, finite and > 0.
 *   q_dtype       PKV_F16 or PKV_BF16 for q and out.
 *   cache_dtype   q_dtype, PKV_FP8_E4M3 or PKV_INT8 (others are
 *                 PKV_ERR_UNSUPPORTED); D and BS as for the decode.
 *   k_scale, v_scale  8-bit pool scales, finite and > 0 (ignored otherwise).
 * Rows of a sequence whose q_s breaks q_s <= min(n_s, max_q_len) are partly
 * left unwritten; cu_q_lens entries are clamped into [0, Tq], so no access
 * leaves the buffers.  S, Tq or max_q_len = 0 is a no-op that returns PKV_OK.
 * Needs no workspace.
 */
pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* cu_q_lens, int32_t S,
                                       int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS,
                                       int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
                                       pkv_dtype cache_dtype, float k_scale, float v_scale, hipStream_t stream);

/*
 * A prompt step's cache write and prompt attention in one pass: the new
 * tokens' K/V are stored in the blocks their sequences map and attended
 * together with the cached context ([P2] §2.1 step 1: a prompt's K/V are
 * stored block by block and used; [P3] §2.2: the slots come from the slot
 * mapping).  Equivalent, bit for bit in out and in both pools, to
 *   pkv_reshape_and_cache(key, value, ..., slot_mapping, T = Tq, ...)
 *   pkv_paged_attention_prefill(out, q, ...)
 * For F16/BF16 pools without a separate write kernel: each workgroup stores
 * its own new tokens, and the attention reads every new token's K/V from
 * key / value (only the cached context through the block tables).  For
 * 8-bit pools the cache-write kernel runs first (it quantises), and writes
 * every token with a non-negative slot.
 *   key, value    [Tq][H][D] q_dtype, 16-byte aligned: the new tokens, packed
 *                 by sequence as q is (cu_q_lens).
 *   slot_mapping  int32 [Tq]: the slot of new token i of sequence s must be
 *                 the slot of position context_lens[s] - q_s + i (q_s its
 *                 count of new tokens), or negative to skip its write.
 *                 New tokens beyond context_lens[s] and tokens outside every
 *                 sequence's range are not written.  Otherwise the pools
 *                 still receive the writes, but the output is unspecified.
 * Other arguments and checks as for pkv_paged_attention_prefill.
 */
pkv_status pkv_paged_attention_prefill_append(void* out, const void* q, const void* key, const void* value,
                                              void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              const int32_t* cu_q_lens, int32_t S, int32_t Tq,
                                              int32_t max_q_len, int32_t H, int32_t D, int32_t BS, int32_t MB,
                                              int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                              float k_scale, float v_scale, hipStream_t stream);

/* The prompt attention and its appending form with one scale per head of
 * each 8-bit pool (k_scales / v_scales fp32 [H] on the device, in place of
 * k_scale / v_scale); everything else as for pkv_paged_attention_prefill
 * and pkv_paged_attention_prefill_append. */
pkv_status pkv_paged_attention_prefill_head_scales(void* out, const void* q, const void* k_cache,
                                                   const void* v_cache, const int32_t* block_tables,
                                                   const int32_t* context_lens, const int32_t* cu_q_lens, int32_t S,
                                                   int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS,
                                                   int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
                                                   pkv_dtype cache_dtype, const float* k_scales,
                                                   const float* v_scales, hipStream_t stream);

pkv_status pkv_paged_attention_prefill_append_head_scales(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens,
    int32_t S, int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, const float* k_scales, const float* v_scales, hipStream_t stream);

/*
 * Copy-on-write block copies ([P2] §2.2): for each of the N pairs
 * (src, dst) = (pairs[2i], pairs[2i+1]), block dst of both pools becomes a
 * bitwise copy of block src (all heads).  pairs is int32 [N][2] on the device.
 * N = 0 is a no-op that returns PKV_OK.
 */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t N,
                           int32_t H, int32_t D, int32_t BS, int32_t NB, pkv_dtype cache_dtype,
                           hipStream_t stream);

/*
 * Move whole blocks between two pool pairs, typically the GPU pools and a
 * swap space in pinned host memory, either way round ([P1] §4.1: the
 * swap-space flag; [P2] §5.2: when GPU memory runs short, part of the KV
 * cache moves to CPU memory, which costs speed but lifts the memory limit).
 * For each of the N pairs (src, dst) = (pairs[2i], pairs[2i+1]), block dst of
 * the destination pools becomes a bitwise copy of block src of the source
 * pools (all heads, K and V).
 *   dst_k_cache, dst_v_cache  [NB_dst][H][BS][D] cache_dtype (written).
 *   src_k_cache, src_v_cache  [NB_src][H][BS][D] cache_dtype.
 *   pairs         int32 [N][2].
 * Every pointer must be device memory or pinned host memory (hipHostMalloc);
 * anything else, such as pageable host memory, is PKV_ERR_INVALID_ARG and
 * nothing is enqueued.  The copy is one kernel that reaches the host side
 * over the host link.  A pair naming a block outside its pool is skipped; a
 * repeated destination gives an unspecified result.  The host side may be
 * read only after the stream has passed the call.  N = 0 is a no-op that
 * returns PKV_OK.
 */
pkv_status pkv_swap_blocks(void* dst_k_cache, void* dst_v_cache, const void* src_k_cache,
                           const void* src_v_cache, const int32_t* pairs, int32_t N, int32_t H, int32_t D,
                           int32_t BS, int32_t NB_src, int32_t NB_dst, pkv_dtype cache_dtype,
                           hipStream_t stream);

/*
 * The decode's block gather on its own ([P2] §2.1), exported for testing:
 * k_out[cu_lens[s] + t][h][:] = k_cache[block_tables[s][t / BS]][h][t % BS][:]
 * for t < context_lens[s], likewise v_out; raw bits are copied.  It uses
 * the same device address computation as the decode kernel.
 *   k_out, v_out  [cu_lens[S]][H][D] cache_dtype (written).
 *   cu_lens       int32 [S + 1] on the device, cu_lens[0] = 0,
 *                 cu_lens[s + 1] = cu_lens[s] + context_lens[s]; the caller
 *                 owns its consistency with k_out's size.
 */
pkv_status pkv_gather_kv(void* k_out, void* v_out, const int32_t* cu_lens, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS,
                         int32_t MB, int32_t NB, pkv_dtype cache_dtype, hipStream_t stream);

/*
 * Read-only bandwidth probe, exported for measurement: reads every 16-byte
 * chunk of buf once, with the same non-temporal 16-byte loads as the decode's
 * K/V stream; each wave reads contiguous 8 KiB spans, eight wave-wide 1 KiB
 * loads in flight.  Its rate is the achievable sequential read bandwidth of
 * the device, set beside the decode's K/V rate as a second denominator to
 * the published peak.
 *   buf    device memory, 16-byte aligned; its contents do not matter.
 *   bytes  a multiple of 16 (else PKV_ERR_INVALID_ARG); 0 is a no-op.
 *   sink   one device uint32, 4-byte aligned.  It is written only when the
 *          XOR of the words one lane read equals 0x9e3779b9 (so the loads
 *          cannot be optimised away), and then holds that value.
 */
pkv_status pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * HIP-graph capture of the decode step ([P3] §3: the decode step is captured
 * once over input buffers of a fixed maximum batch size and replayed every
 * step, which removes most of its launch overhead).  The step is: the
 * copy-on-write copies (if num_pairs > 0), the cache write of one new token
 * per batch slot, and the decode (both phases), exactly as the eager calls
 * pkv_copy_blocks, pkv_reshape_and_cache, pkv_paged_attention_decode_partitions
 * and pkv_paged_attention_decode_merge with these arguments would enqueue it.
 *
 * Every pointer below names a fixed device buffer owned by the caller; it
 * must stay allocated, at the same address, until the graph is destroyed.
 * Each launch reads and writes the buffers' current contents, so the caller
 * moves to the next step by rewriting them (new tokens, slot_mapping,
 * block_tables, context_lens, q, copy_pairs) on the launch stream or before
 * it.  Sizes, dtypes and the three scales are fixed at capture.  A batch slot
 * without a sequence carries slot_mapping = -1 (nothing written) and
 * context_lens = 0 (zero output); an unused copy pair carries ids outside
 * [0, NB) (skipped).
 *
 * The graph is an object created and destroyed by the caller; it is tied to
 * the device that is current at creation.  Two launches of one graph must
 * not overlap.  Capture uses a private stream of default priority; nothing
 * recorded is a memset.
 */
typedef struct pkv_decode_graph pkv_decode_graph;

typedef struct {
  void* k_cache;                /* [NB][H][BS][D] cache_dtype */
  void* v_cache;
  const void* key;              /* [S][H][D] q_dtype: each batch slot's new token */
  const void* value;
  const int32_t* slot_mapping;  /* int32 [S] */
  const int32_t* copy_pairs;    /* int32 [num_pairs][2] (src, dst), applied first */
  int32_t num_pairs;            /* >= 0 */
  const void* q;                /* [S][H][D] q_dtype */
  void* out;                    /* [S][H][D] q_dtype */
  const int32_t* block_tables;  /* int32 [S][MB] */
  const int32_t* context_lens;  /* int32 [S] */
  void* workspace;              /* pkv_decode_workspace_bytes(S, H, D, BS, MB) bytes */
  size_t workspace_bytes;
  int32_t S, H, D, BS, MB, NB;
  float scale, k_scale, v_scale;
  pkv_dtype q_dtype, cache_dtype;
  int32_t append;               /* nonzero: the cache write and the decode are
                                   recorded as pkv_paged_attention_decode_append
                                   (its contract on slot_mapping applies);
                                   0: as the separate calls */
  const float* k_scales;        /* 8-bit pools with one scale per head: fp32 [H]
                                   device arrays, read at every replay; the calls
                                   are recorded in their *_head_scales forms and
                                   k_scale / v_scale are ignored.  NULL: one
                                   scale per pool. */
  const float* v_scales;
} pkv_decode_step;

/* Capture the step into a new graph.  Every check of the eager calls applies
 * (with their status codes); on failure *graph is NULL and nothing stays
 * allocated.  S must be > 0.  Synchronous with respect to the host; enqueues
 * no work. */
pkv_status pkv_decode_graph_create(const pkv_decode_step* step, pkv_decode_graph** graph);

/* Enqueue one replay of the captured step on `stream` (NULL = the null stream). */
pkv_status pkv_decode_graph_launch(pkv_decode_graph* graph, hipStream_t stream);

/* Free the graph (NULL is a no-op).  Replays already enqueued still run; the
 * caller synchronises before reusing the buffers for anything else. */
pkv_status pkv_decode_graph_destroy(pkv_decode_graph* graph);

/*
 * Device-side check of one step's index inputs, for debugging a caller's
 * block bookkeeping: the block tables and context lengths ([P1] §2.2,
 * [P2] §2.1), the slot mapping of the new tokens ([P3] §2.2) and the
 * copy-on-write pairs ([P2] §2.2).  The compute calls above stay inside
 * their buffers whatever these hold, but give unspecified results when one
 * of the following conditions is broken; this call reports which, as a mask
 * of pkv_check_bit values:
 */
typedef enum {
  PKV_CHECK_CONTEXT_LEN = 1 << 0,   /* a context length outside [0, MB*BS] */
  PKV_CHECK_BLOCK_ID = 1 << 1,      /* a used table entry (logical block
                                       j < ceil(n_s / BS), n_s clamped into
                                       [0, MB*BS]) outside [0, NB) */
  PKV_CHECK_SLOT_RANGE = 1 << 2,    /* a slot >= NB*BS (negative = padding) */
  PKV_CHECK_SLOT_DUP = 1 << 3,      /* two tokens name one slot */
  PKV_CHECK_PAIR_RANGE = 1 << 4,    /* a copy pair names a block outside [0, NB) */
  PKV_CHECK_PAIR_OVERLAP = 1 << 5,  /* copy destinations repeat, or a
                                       destination is also a source */
  PKV_CHECK_APPEND_SLOT = 1 << 6,   /* append != 0 only: a sequence's slot is
                                       not that of its position n_s - 1
                                       through its table, or n_s = 0 with a
                                       slot given ([P2] §2.1) */
  PKV_CHECK_SHARED_WRITE = 1 << 7   /* a written slot lies in a block that
                                       more than one used table entry maps:
                                       the block had to be copied first
                                       ([P2] §2.2) */
} pkv_check_bit;

/* Bytes of device workspace pkv_check_step_inputs needs for a pool of NB
 * blocks of BS tokens (0 for non-positive sizes): 256 B, then NB*BS bits of
 * slot bitmap, 2*NB bits of copy bitmaps and NB 32-bit map counts, each
 * section rounded up to 256 B.  C4-sized pools (about 1,000 blocks of 16)
 * need about 7 KiB; a 12,400-block pool of 32 about 100 KiB. */
size_t pkv_check_workspace_bytes(int32_t NB, int32_t BS);

/*
 * Check the index inputs of one step against the conditions above.
 *   block_tables  int32 [S][MB], context_lens int32 [S] (both may be NULL
 *                 when S == 0).
 *   slot_mapping  int32 [T], the step's new tokens (NULL when T == 0).
 *   pairs         int32 [N][2] copy-on-write (src, dst) pairs (NULL when
 *                 N == 0).
 *   append        nonzero: the step is an appending decode, one new token
 *                 per sequence (T must equal S), and PKV_CHECK_APPEND_SLOT
 *                 is checked too.
 *   workspace     device memory of pkv_check_workspace_bytes(NB, BS) bytes
 *                 or more, 4-byte aligned; overwritten.
 *   violations    host pointer that receives the mask (may be NULL).
 * Returns PKV_OK when the mask is 0 and PKV_ERR_DEVICE_CHECK otherwise.
 * Unlike every other call it synchronises `stream` (it reads the mask back),
 * so it cannot be captured into a graph.  Argument errors return
 * PKV_ERR_INVALID_ARG (S, T, N < 0, MB, BS, NB <= 0, a needed pointer NULL,
 * append with T != S) or PKV_ERR_WORKSPACE; HIP failures PKV_ERR_HIP.
 */
pkv_status pkv_check_step_inputs(const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t MB,
                                 const int32_t* slot_mapping, int32_t T, const int32_t* pairs, int32_t N,
                                 int32_t BS, int32_t NB, int32_t append, void* workspace,
                                 size_t workspace_bytes, uint32_t* violations, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */

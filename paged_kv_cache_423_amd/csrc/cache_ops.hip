// Cache-side kernels for gfx950: the slot-mapping write of new tokens' K/V,
// copy-on-write block copies, and the block gather exported for testing.
//
// Cache write: the int32 slot mapping names each new token's slot, numbered
// block * block_size + offset (l189.com article on KV cache and
// PagedAttention, www.l189.com/news/180929, §2.2); the generated token's K/V
// go into the block its sequence maps ("在A10G上榨干LLaMA-7B：vLLM与
// PagedAttention实战" §2.1).  Block copies implement the copy step of
// copy-on-write (same page, §2.2).
//
// All three kernels move 16-byte chunks per lane over contiguous runs, so
// every wave-wide access covers whole 1 KiB spans of a row-contiguous layout.

#include "device_common.h"
#include "kernels.h"

namespace pkv {

constexpr int kCacheThreads = 256;

// Two fp32 values -> two OCP E4M3FN bytes (bits 0-15 of the result): round
// to nearest even, saturating to +-448 (infinities included), NaN -> 0x7F.
// gfx950's conversion instruction encodes OCP E4M3FN with round to nearest
// even, subnormals included; it would turn an overflow into NaN, so the
// values are clamped into [-448, 448] first (which changes no result: every
// value past 448 saturates), and a NaN input, which the clamp turned into a
// number, gets the one NaN code the format reading fixes.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2_sat_rn(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.0f), 448.0f);
  const float cb = fminf(fmaxf(b, -448.0f), 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  if (a != a) r = (r & 0xFF00u) | 0x7Fu;
  if (b != b) r = (r & 0x00FFu) | 0x7F00u;
  return r;
}

// fp32 -> INT8 byte: nearest integer, ties to even, saturated to [-127, 127]
// (infinities included); NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_i8_sat_rn(float x) {
  if (x != x) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(x, -127.0f), 127.0f));
  return (uint32_t)(int32_t)r & 0xFFu;
}

// One 16-byte chunk of a new token's key or value row (16 / bytes(SFMT)
// elements) written into a [NB][H][BS][D] pool at element index dst: a bit
// copy when the formats match, else every element divided by the pool's
// scale (IEEE fp32 division, round to nearest even) and encoded in the
// 8-bit format with saturation.
template <int SFMT, int CFMT>
__device__ __forceinline__ void write_cache_chunk(void* pool, size_t dst, const u32x4& src, float scale) {
  constexpr int CB = FmtInfo<CFMT>::bytes;
  if constexpr (SFMT == CFMT) {
    store16((char*)pool + dst * CB, src);
  } else {
    static_assert(scaled_format(CFMT) && FmtInfo<SFMT>::bytes == 2, "16-bit sources quantise to an 8-bit format");
    float f[8];
    Chunk<SFMT>::to_f32(src, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __fdiv_rn(f[i], scale);
    uint32_t w[2] = {0u, 0u};
    if constexpr (CFMT == E4M3) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) w[i >> 2] |= f32x2_to_e4m3x2_sat_rn(f[i], f[i + 1]) << (8 * (i & 3));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i >> 2] |= f32_to_i8_sat_rn(f[i]) << (8 * (i & 3));
    }
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2_t*>((char*)pool + dst) = u32x2_t{w[0], w[1]};
  }
}

// One workgroup per new token; lane c moves chunk c, c + 256, ... of the
// token's H*D row block of K and of V.  A chunk is 16 source bytes.  8-bit
// pools divide by the pool's scale, or by the chunk's head's scale when
// k_scales / v_scales are given.
template <int SFMT, int CFMT>
__global__ __launch_bounds__(kCacheThreads) void reshape_and_cache_kernel(
    const void* __restrict__ key, const void* __restrict__ value, void* __restrict__ k_cache,
    void* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int H, int D, int BS,
    int NB, float k_scale, float v_scale, const float* __restrict__ k_scales, const float* __restrict__ v_scales) {
  constexpr int SB = FmtInfo<SFMT>::bytes;
  constexpr int EPC = 16 / SB;                 // source elements per chunk
  const int t = blockIdx.x;
  const int slot = slot_mapping[t];
  // negative: padding token; past the pool: skipped so that no write leaves it
  if (slot < 0 || slot / BS >= NB) return;
  const int blk = slot / BS, off = slot % BS;
  const int cpr = D / EPC;                     // chunks per head row
  const int nchunks = H * cpr;
  const char* ksrc = (const char*)key + (size_t)t * H * D * SB;
  const char* vsrc = (const char*)value + (size_t)t * H * D * SB;
  for (int c = threadIdx.x; c < nchunks; c += kCacheThreads) {
    const int h = c / cpr;
    const int e0 = (c % cpr) * EPC;
    const size_t src = ((size_t)h * D + e0) * SB;
    const size_t dst = (((size_t)blk * H + h) * BS + off) * D + e0;   // elements
    float ks = k_scale, vs = v_scale;
    if constexpr (SFMT != CFMT) {
      if (k_scales) ks = k_scales[h];
      if (v_scales) vs = v_scales[h];
    }
    write_cache_chunk<SFMT, CFMT>(k_cache, dst, load16(ksrc + src), ks);
    write_cache_chunk<SFMT, CFMT>(v_cache, dst, load16(vsrc + src), vs);
  }
}

// grid.x = 2 * pair (even: K pool, odd: V pool), grid.y splits one block's
// bytes; each workgroup copies a contiguous span in 16-byte chunks.
constexpr int kCopyChunksPerThread = 4;
constexpr size_t kCopySpan = (size_t)kCacheThreads * 16 * kCopyChunksPerThread;

__global__ __launch_bounds__(kCacheThreads) void copy_blocks_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache, const int32_t* __restrict__ pairs,
    int NB, size_t block_bytes) {
  const int pair = blockIdx.x >> 1;
  char* pool = (blockIdx.x & 1) ? (char*)v_cache : (char*)k_cache;
  const int64_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if ((uint64_t)src >= (uint64_t)NB || (uint64_t)dst >= (uint64_t)NB) return;   // out of the pool: skipped
  const char* from = pool + (size_t)src * block_bytes;
  char* to = pool + (size_t)dst * block_bytes;
  const size_t begin = (size_t)blockIdx.y * kCopySpan;
  const size_t end = begin + kCopySpan < block_bytes ? begin + kCopySpan : block_bytes;
  u32x4 buf[kCopyChunksPerThread];
#pragma unroll
  for (int i = 0; i < kCopyChunksPerThread; ++i) {
    const size_t o = begin + ((size_t)i * kCacheThreads + threadIdx.x) * 16;
    if (o < end) buf[i] = load16(from + o);
  }
  // non-temporal stores: with plain ones, which leave the copies as dirty
  // lines in the caches, the decode that follows the copies of the
  // shared-prefix step ran about 11% slower
#pragma unroll
  for (int i = 0; i < kCopyChunksPerThread; ++i) {
    const size_t o = begin + ((size_t)i * kCacheThreads + threadIdx.x) * 16;
    if (o < end) __builtin_nontemporal_store(buf[i], reinterpret_cast<u32x4*>(to + o));
  }
}

// Block swap between two pools (a GPU cache and a swap space in pinned host
// memory, either way round: "vLLM-v0.17.1技术解析" §4.1, the swap-space flag;
// "在A10G上榨干LLaMA-7B" §5.2, KV blocks moved to CPU memory when GPU memory
// runs short).  Same split as copy_blocks_kernel; the host side is reached
// over the host link, so each lane keeps four 16-byte accesses in flight.
__global__ __launch_bounds__(kCacheThreads) void swap_blocks_kernel(
    void* __restrict__ dst_k, void* __restrict__ dst_v, const void* __restrict__ src_k,
    const void* __restrict__ src_v, const int32_t* __restrict__ pairs, int NB_src, int NB_dst,
    size_t block_bytes) {
  const int pair = blockIdx.x >> 1;
  const bool is_v = blockIdx.x & 1;
  const char* src_pool = (const char*)(is_v ? src_v : src_k);
  char* dst_pool = (char*)(is_v ? dst_v : dst_k);
  const int64_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if ((uint64_t)src >= (uint64_t)NB_src || (uint64_t)dst >= (uint64_t)NB_dst) return;   // skipped
  const char* from = src_pool + (size_t)src * block_bytes;
  char* to = dst_pool + (size_t)dst * block_bytes;
  const size_t begin = (size_t)blockIdx.y * kCopySpan;
  const size_t end = begin + kCopySpan < block_bytes ? begin + kCopySpan : block_bytes;
  u32x4 buf[kCopyChunksPerThread];
#pragma unroll
  for (int i = 0; i < kCopyChunksPerThread; ++i) {
    const size_t o = begin + ((size_t)i * kCacheThreads + threadIdx.x) * 16;
    if (o < end) buf[i] = *reinterpret_cast<const u32x4*>(from + o);
  }
#pragma unroll
  for (int i = 0; i < kCopyChunksPerThread; ++i) {
    const size_t o = begin + ((size_t)i * kCacheThreads + threadIdx.x) * 16;
    if (o < end) store16(to + o, buf[i]);
  }
}

// One workgroup per (logical block j, sequence s): rows t of block j with
// t < n_s, every head, to k_out[cu_lens[s] + t].  Addresses come from the
// same tile_base rule as the decode kernel.
template <int CFMT, int D, int BS>
__global__ __launch_bounds__(kCacheThreads) void gather_kv_kernel(
    void* __restrict__ k_out, void* __restrict__ v_out, const int32_t* __restrict__ cu_lens,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, int H,
    int MB, int NB) {
  constexpr int EB = FmtInfo<CFMT>::bytes;
  constexpr int EPC = 16 / EB;
  constexpr int CPR = D / EPC;                 // chunks per row
  const int j = blockIdx.x;
  const int s = blockIdx.y;
  const int n = min(max(context_lens[s], 0), MB * BS);
  const int rows = min(BS, n - j * BS);
  if (rows <= 0) return;
  int64_t phys = block_tables[(size_t)s * MB + j];
  if ((uint64_t)phys >= (uint64_t)NB) phys = 0;      // out-of-range id: stay inside the pool
  const size_t row0 = (size_t)cu_lens[s] + (size_t)j * BS;
  const int nchunks = H * rows * CPR;
  for (int c = threadIdx.x; c < nchunks; c += kCacheThreads) {
    const int col = c % CPR;
    const int r = (c / CPR) % rows;
    const int h = c / (CPR * rows);
    const size_t src = (tile_base<D, BS>(phys, h, H) + (size_t)r * D + (size_t)col * EPC) * EB;
    const size_t dst = (((row0 + r) * H + h) * D + (size_t)col * EPC) * EB;
    store16((char*)k_out + dst, load16((const char*)k_cache + src));
    store16((char*)v_out + dst, load16((const char*)v_cache + src));
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int T, int H, int D, int BS, int NB,
                                    int src_fmt, int c_fmt, float k_scale, float v_scale,
                                    const float* k_scales, const float* v_scales, hipStream_t st) {
  dim3 grid(T), block(kCacheThreads);
#define PKV_RC(S_, C_)                                                                         \
  hipLaunchKernelGGL((reshape_and_cache_kernel<S_, C_>), grid, block, 0, st, key, value, k_cache, \
                     v_cache, slot_mapping, H, D, BS, NB, k_scale, v_scale, k_scales, v_scales)
  if (src_fmt == F32 && c_fmt == F32) PKV_RC(F32, F32);
  else if (src_fmt == F16 && c_fmt == F16) PKV_RC(F16, F16);
  else if (src_fmt == BF16 && c_fmt == BF16) PKV_RC(BF16, BF16);
  else if (src_fmt == F16 && c_fmt == E4M3) PKV_RC(F16, E4M3);
  else if (src_fmt == BF16 && c_fmt == E4M3) PKV_RC(BF16, E4M3);
  else if (src_fmt == F16 && c_fmt == I8) PKV_RC(F16, I8);
  else if (src_fmt == BF16 && c_fmt == I8) PKV_RC(BF16, I8);
  else return hipErrorInvalidValue;
#undef PKV_RC
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int N, int NB,
                              size_t block_bytes, hipStream_t st) {
  const unsigned spans = (unsigned)((block_bytes + kCopySpan - 1) / kCopySpan);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(2 * N, spans), dim3(kCacheThreads), 0, st, k_cache,
                     v_cache, pairs, NB, block_bytes);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int N, int NB_src, int NB_dst, size_t block_bytes,
                              hipStream_t st) {
  const unsigned spans = (unsigned)((block_bytes + kCopySpan - 1) / kCopySpan);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(2 * N, spans), dim3(kCacheThreads), 0, st, dst_k, dst_v, src_k,
                     src_v, pairs, NB_src, NB_dst, block_bytes);
  return hipGetLastError();
}

template <int CFMT>
static hipError_t gather_c(void* k_out, void* v_out, const int32_t* cu, const void* kc, const void* vc,
                           const int32_t* bt, const int32_t* cl, int S, int H, int D, int BS, int MB,
                           int NB, hipStream_t st) {
  dim3 grid(MB, S), block(kCacheThreads);
#define PKV_G(D_, BS_)                                                                            \
  hipLaunchKernelGGL((gather_kv_kernel<CFMT, D_, BS_>), grid, block, 0, st, k_out, v_out, cu, kc, vc, \
                     bt, cl, H, MB, NB)
#define PKV_GD(D_) \
  if (D == D_) { if (BS == 16) PKV_G(D_, 16); else PKV_G(D_, 32); return hipGetLastError(); }
  PKV_GD(64) PKV_GD(80) PKV_GD(96) PKV_GD(128) PKV_GD(256)
#undef PKV_GD
#undef PKV_G
  return hipErrorInvalidValue;
}

hipError_t launch_gather_kv(void* k_out, void* v_out, const int32_t* cu_lens, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int S, int H, int D, int BS, int MB,
                            int NB, int c_fmt, hipStream_t st) {
  switch (c_fmt) {
    case F32: return gather_c<F32>(k_out, v_out, cu_lens, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, st);
    case F16: return gather_c<F16>(k_out, v_out, cu_lens, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, st);
    case BF16: return gather_c<BF16>(k_out, v_out, cu_lens, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, st);
    case I8:
    case E4M3: return gather_c<E4M3>(k_out, v_out, cu_lens, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, st);
    default: return hipErrorInvalidValue;
  }
}

// Read-only bandwidth probe: the achievable HBM read rate for a plain
// sequential stream on this device, to set beside the decode's rate.  Each
// 16-byte chunk of the buffer is read once with the same non-temporal load
// as the decode's K/V stream.  A wave reads a contiguous span of
// kStreamInFlight KiB per pass (that many wave-wide 1 KiB loads in flight),
// the waves of the grid take consecutive spans.  Spans keep DRAM pages
// together: the same eight loads per lane spread one grid-width apart read
// about 15% slower.  The XOR of what a lane read is stored to *sink only
// when it equals kStreamMark, so the loads cannot be dropped and nothing
// else is written.
constexpr int kStreamThreads = 256;
constexpr int kStreamInFlight = 8;
constexpr int kStreamBlocks = 4096;           // 16 workgroups of 4 waves per CU
constexpr uint32_t kStreamMark = 0x9e3779b9u;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const char* __restrict__ buf,
                                                                     size_t chunks, uint32_t* __restrict__ sink) {
  constexpr size_t span = 64 * kStreamInFlight;                  // chunks per wave and pass
  const size_t lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6);
  const size_t nwaves = (size_t)gridDim.x * (kStreamThreads / 64);
  uint32_t x = 0;
  for (size_t base = wave * span; base < chunks; base += nwaves * span) {
    u32x4 v[kStreamInFlight];
#pragma unroll
    for (int i = 0; i < kStreamInFlight; ++i) {
      const size_t c = base + (size_t)i * 64 + lane;
      v[i] = c < chunks ? load16(buf + c * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kStreamInFlight; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  if (x == kStreamMark) *sink = x;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  stream_read_kernel<<<kStreamBlocks, kStreamThreads, 0, st>>>((const char*)buf, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv

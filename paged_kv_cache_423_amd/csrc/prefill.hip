// Multi-query paged attention for gfx950: the new tokens of each sequence (a
// prompt, or the part of a prompt past a cached shared prefix) attend
// causally over the sequence's K/V in fixed-size physical blocks reached
// through its block table ("在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战"
// §2.1 step 1 and §2.2: a prompt's K/V are stored block by block and then
// used; a shared prompt prefix is stored once).  New token i of a sequence
// that holds n tokens, q of them new, sits at position n - q + i and sees
// positions 0 .. n - q + i.
//
// Unlike the single-query decode this is a dense contraction (QK^T and PV
// with 32 queries sharing every key), so it runs on the matrix cores
// ("vLLM-v0.17.1技术解析" §3.2 names a fused FlashAttention-style kernel; this
// one is written for CDNA4's MFMA instead).
//
// Work split.  One workgroup of 4 wave64s takes 128 consecutive new tokens of
// one (head, sequence), aligned to the end of the sequence's new tokens so
// that the first workgroups carry the longest key ranges.  Each wave owns 32
// queries.  Keys are consumed in tiles of 32 tokens that go from global memory
// straight into LDS (double-buffered, one barrier per tile; details below).
//
// Per tile and wave (v_mfma_f32_32x32x16, fp32 accumulate):
//   S^T[key][query]  = K . Q^T      (D/16 MFMAs; Q^T stays in registers)
//   online softmax over the keys: each lane holds one query column and 16
//   keys of it, the other 16 in lane ^ 32
//   O^T[d][query]   += V^T . P^T    (D/32 x 2 MFMAs; P rounded to the
//                                    operand format)
// The accumulator of S^T holds, in lane l, query l % 32 and keys
// 8j + 4(l / 32) + i (j, i < 4); used as the B operand of the second product,
// its 8 values per 16-key chunk c are the keys 16c + 4(l / 32) + {0..3} and
// 16c + 8 + 4(l / 32) + {0..3}, so the V^T operand of the same lane reads
// exactly those keys: the order of the contraction over keys is permuted
// consistently on both sides.  The V^T operand is read out of a row-major V
// tile with a transposing LDS read.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int FMT> struct Mma;
template <> struct Mma<BF16> {
  __device__ __forceinline__ static f32x16 mac(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
  // two fp32 -> packed pair of the operand format, round to nearest even
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
  }
  // acc + the two values of a packed pair (v_dot2 with (1, 1))
  __device__ __forceinline__ static float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                           acc, false);
  }
  // two E4M3 bytes of w (bytes 0-1, or 2-3 when HI) -> packed pair, exact
  // (one gfx950 conversion; a scale of 1 leaves the values unchanged)
  template <bool HI>
  __device__ __forceinline__ static uint32_t from_e4m3(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
};
template <> struct Mma<F16> {
  __device__ __forceinline__ static f32x16 mac(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2));
  }
  __device__ __forceinline__ static float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
  }
  template <bool HI>
  __device__ __forceinline__ static uint32_t from_e4m3(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
};

// Workgroups per CU the register budget is sized for (3: 163 VGPRs at
// D = 128; 4 spills).
constexpr int kPfMinWg = 3;

constexpr int kPfWaves = 4;                  // waves per workgroup
constexpr int kPfQW = 32;                    // queries per wave
constexpr int kPfQT = kPfWaves * kPfQW;      // queries per workgroup
constexpr int kPfKT = 32;                    // keys per tile (one 32-row block of S^T)
constexpr int kPfBufs = 2;                   // LDS tile buffers: tile k + 1 loads while tile k is used
constexpr float kSlack = 8.0f;               // softmax weights stay below 2^kSlack

__device__ __forceinline__ u32x4 load16_cached(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// The two halves of a wave hold the same query columns; v_permlane32_swap
// hands every lane its partner's value (lane ^ 32) without going through LDS.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// The key tiles go from global memory straight into LDS (global_load_lds_
// dwordx4: no staging registers, no LDS stores), K and V both row-major; the
// V^T operand comes from the transposing LDS read ds_read_b64_tr_b16.  Within
// each group of 16 lanes that read returns to lane
// j the element j % 4 of the 8-byte reads of lanes j / 4, 4 + j / 4,
// 8 + j / 4 and 12 + j / 4: when lane s = 4k + m of the group reads row
// t0 + k, columns c0 + 4m .. c0 + 4m + 3, lane j receives V[t0 .. t0 + 3][c0 + j].
//
// LDS image of one tile of one tensor: 32 rows of RB = 2D bytes, no padding
// (a direct load writes 16 * 64 consecutive bytes per wave); 16-byte chunk c
// of row t sits at chunk position c ^ swz(t).  gfx950's LDS serves 256 bytes
// (64 banks) per cycle, so a conflict-free read spreads 16 lanes' 16-byte
// operands, or 32 lanes' 8-byte transposing reads, over 16 different chunk
// slots: K by t mod 16 (sixteen rows at one chunk), V by 4 (t mod 4) (four
// rows times four chunks per 32 lanes).  Rows of 8 chunks (D = 64) use
// t mod 8 and 2 (t mod 4); head sizes whose row has a non-power-of-two
// number of chunks (80, 96) are not swizzled.
template <int D>
struct PfSwz {
  static constexpr int DC = D / 8;
  static constexpr bool on = (DC & (DC - 1)) == 0 && DC >= 8;
  static constexpr bool wide = on && DC >= 16;     // rows of 16 or more chunks
  __device__ __forceinline__ static int k(int t) { return on ? (t & (wide ? 15 : 7)) : 0; }
  __device__ __forceinline__ static int v(int t) { return on ? (wide ? 4 : 2) * (t & 3) : 0; }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 bytes from global address g into LDS at dst + 16 * lane (dst uniform
// over the wave): global_load_lds_dwordx4.
__device__ __forceinline__ void load16_to_lds(const void* g, char* dst) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// x, opaque to the optimiser.  A direct load's address, a uniform 64-bit
// base plus a lane offset fixed for the whole loop, then stays in that form
// (the scalar-base load with a 32-bit vector offset): otherwise the compiler
// adds each lane offset to the pool pointer once before the loop and keeps
// the 64-bit sums in vector registers throughout it.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// ds_read_b64_tr_b16 at p (see above): four 16-bit values as two words.
__device__ __forceinline__ u32x2 lds_read_tr16x4(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Sixteen 8-bit pool values (one 16-byte load) as two 16-byte chunks of the
// operand format FMT: elements 0-7 and 8-15, exact.  E4M3 bytes convert two
// at a time straight to the operand format.  An INT8 byte b comes out as
// b + 128 (0 .. 255, exact in both operand formats); the kernel takes the
// offset off once per query instead of once per element: 128 * sum(q) from
// each score and 128 * sum(p) from each output.
template <int FMT, int CFMT>
__device__ __forceinline__ void to_operand(const u32x4& c, u32x4& lo, u32x4& hi) {
  if constexpr (CFMT == E4M3) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      lo[2 * w] = Mma<FMT>::template from_e4m3<false>(c[w]);
      lo[2 * w + 1] = Mma<FMT>::template from_e4m3<true>(c[w]);
      hi[2 * w] = Mma<FMT>::template from_e4m3<false>(c[2 + w]);
      hi[2 * w + 1] = Mma<FMT>::template from_e4m3<true>(c[2 + w]);
    }
  } else {
    float f[16];
    Chunk<CFMT>::to_f32(c, f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      lo[w] = Mma<FMT>::pack(f[2 * w], f[2 * w + 1]);
      hi[w] = Mma<FMT>::pack(f[8 + 2 * w], f[8 + 2 * w + 1]);
    }
  }
}

// APPEND: the new tokens' K/V are stored into the pools by this kernel (each
// workgroup its own query range), and the tiles read them from new_k /
// new_v instead of from the pools (see below).
//
// CFMT: the pools' format.  F16 / BF16 pools (CFMT == FMT) go into LDS with
// direct loads.  8-bit pools (E4M3, INT8) are loaded into registers one tile
// ahead, converted to FMT (exactly: every E4M3 and INT8 value is a bf16 and
// an fp16 value) and stored into the same LDS image after the current tile's
// products; their scales are folded into s_mult (k_scale) and out_mult
// (v_scale), as in the decode.
template <int FMT, int CFMT, int D, int BS, bool APPEND>
__global__ __launch_bounds__(kPfWaves * 64, D >= 256 ? 1 : kPfMinWg) void paged_prefill_kernel(
    void* __restrict__ out, const void* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens, int Tq, int H, int MB,
    int NB, float s_mult, float out_mult, const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const void* __restrict__ new_k, const void* __restrict__ new_v, const int32_t* __restrict__ slot_mapping) {
  constexpr bool DIRECT = CFMT == FMT;       // 16-bit pools: tiles go to LDS as they are
  static_assert(DIRECT || scaled_format(CFMT), "pools hold the q format or an 8-bit format");
  static_assert(DIRECT || !APPEND, "8-bit pools get the new tokens from the cache-write kernel");
  constexpr int EB = 2;
  constexpr int RB = D * EB;                 // bytes per token row
  constexpr int DP = (D + 31) / 32 * 32;     // rows of O^T: D rounded up to whole 32-row MFMA tiles
  constexpr int TB = kPfKT * RB;             // bytes of one tile of one tensor
  constexpr int VPAD = (DP - D) * EB;        // the V^T reads of padding rows run this far past the tile
  constexpr int VOFF = TB;                   // V tile after the K tile
  constexpr int BUF = (2 * TB + VPAD + 15) / 16 * 16;
  constexpr int NT = kPfWaves * 64;
  constexpr int ROUNDS = (TB + 16 * NT - 1) / (16 * NT);   // direct-load rounds: 16 bytes per thread each
  constexpr int TB8 = kPfKT * D;             // 8-bit pools: bytes of one tile of one tensor
  constexpr int ROUNDS8 = (TB8 + 16 * NT - 1) / (16 * NT);  // staged 16-byte loads per thread and tensor
  constexpr int KSB = kPfKT / 32;
  constexpr int NBT = kPfKT / BS;
  static_assert(D % 16 == 0, "head size must be a multiple of 16");
  static_assert(kPfKT % 32 == 0 && kPfKT % BS == 0, "tile must be whole 32-key blocks and whole cache blocks");
  using Swz = PfSwz<D>;
  __shared__ __attribute__((aligned(16))) char lds[kPfBufs * BUF];

  const int h = blockIdx.x;
  const int tile = blockIdx.y;
  const int s = blockIdx.z;
  // 8-bit pools with one scale per head: this head's scales multiply the
  // score scale and the output, as the pool's one scale does otherwise
  if constexpr (!DIRECT) {
    if (k_scales) s_mult *= k_scales[h];
    if (v_scales) out_mult *= v_scales[h];
  }
  const int n = min(max(context_lens[s], 0), MB * BS);
  const int qa = min(max(cu_q_lens[s], 0), Tq);
  const int qb = min(max(cu_q_lens[s + 1], qa), Tq);
  const int qn = min(qb - qa, n);            // new tokens (never more than the tokens held)
  const int i_end = qn - tile * kPfQT;       // this workgroup's queries: [i_end - 128, i_end) ∩ [0, qn)
  if (i_end <= 0) return;
  const int i_base = i_end - kPfQT;
  const int pos0 = n - qn;                   // position of new token 0


  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hb = lane >> 5;
  const int wq0 = i_base + wave * kPfQW;     // the wave's first query (may be < 0)
  const int my_q = wq0 + col;
  const bool q_ok = my_q >= 0;
  const int my_pos = pos0 + my_q;
  // last position any query of the wave sees; -1 when the wave holds no
  // query (a workgroup tile reaching before the first new token), so that it
  // skips every tile instead of running over the cached prefix
  const int wave_pos_hi = wq0 + kPfQW - 1 < 0 ? -1 : pos0 + wq0 + kPfQW - 1;
  const int wave_pos_lo = pos0 + max(wq0, 0);
  const int kv_end = pos0 + i_end;           // keys [0, kv_end) are visible to some query here
  const int nkt = (kv_end + kPfKT - 1) / kPfKT;
  const int nblocks = (n + BS - 1) / BS;
  const int32_t* table = block_tables + (size_t)s * MB;

  // Q^T operand: chunk c holds d = 16c + 8hb .. +8 of this lane's query
  u32x4 qop[D / 16];
  {
    const char* qrow = (const char*)q + ((size_t)(qa + (q_ok ? my_q : 0)) * H + h) * D * EB;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qop[c] = q_ok ? load16_cached(qrow + (16 * c + 8 * hb) * EB) : u32x4{0u, 0u, 0u, 0u};
  }
  // INT8 pools: every key element carries + 128, so every score of this
  // query carries 128 * sum(q) too much; in log2 units, qcorr
  float qcorr = 0.0f;
  if constexpr (CFMT == I8) {
    float qs = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) qs = Mma<FMT>::sum2(qop[c][w], qs);
    qcorr = Chunk<I8>::offset * sum_halves(qs) * s_mult;
  }

  f32x16 o[DP / 32];
#pragma unroll
  for (int i = 0; i < DP / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m = -INFINITY;                       // reference for the exponentials (log2 units)
  float l = 0.0f;                            // this lane's part of the running sum
  // what the exponentials subtract (m, or 0 while m = -inf; INT8 pools add
  // qcorr) and the rescale threshold, both changed only where m changes
  auto ref_of = [&](float mv) { return CFMT == I8 ? ((mv == -INFINITY) ? 0.0f : mv) + qcorr
                                                   : (mv == -INFINITY) ? 0.0f : mv; };
  float m_ref = ref_of(m);
  float m_slack = m + kSlack;

  // Physical block ids of one key tile: NBT uniform values, read with scalar
  // loads one tile before the loads that use them.  Ids past the sequence
  // are never read from the table; ids outside the pool read block 0.
  auto tile_ids = [&](int kt, int64_t* ids) {
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
      const int lb = __builtin_amdgcn_readfirstlane(kt * NBT + j);
      int64_t b = lb < nblocks ? (int64_t)table[lb] : 0;
      if ((uint64_t)b >= (uint64_t)NB) b = 0;
      ids[j] = b;
    }
  };

  // This thread's 16-byte slot of the tile image in round r: byte 16 * thread
  // + 16 * NT * r, i.e. row t, chunk position pc; the chunk stored there is
  // pc ^ swz(t) of the row (K and V differ).  Fixed for the whole loop, since
  // a tile is a whole number of blocks.
  // The new tokens' rows (APPEND) are rows of new_k / new_v: a uniform base
  // per tile plus noffk / noffv, this lane's row t times H rows of RB bytes
  // and the same chunk (below 2^32 for any H < 2^18).
  int slot_row[ROUNDS];
  uint32_t offk[ROUNDS], offv[ROUNDS], noffk[ROUNDS], noffv[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int P = 16 * (int)threadIdx.x + 16 * NT * r;
    const int t = P / RB, pc = (P % RB) / 16;
    slot_row[r] = P < TB ? t : kPfKT;        // kPfKT: no slot in this round
    offk[r] = (uint32_t)((t % BS) * RB + 16 * (pc ^ Swz::k(t)));
    offv[r] = (uint32_t)((t % BS) * RB + 16 * (pc ^ Swz::v(t)));
    if constexpr (APPEND) {
      noffk[r] = (uint32_t)t * (uint32_t)H * RB + 16 * (pc ^ Swz::k(t));
      noffv[r] = (uint32_t)t * (uint32_t)H * RB + 16 * (pc ^ Swz::v(t));
    }
  }
  const uint64_t head_bytes = (uint64_t)h * (BS * RB);
  const uint64_t block_bytes = (uint64_t)H * (BS * RB);

  // issue the direct loads of tile kt into buffer buf (rows past n: zeros)
  auto fetch = [&](int kt, int buf, const int64_t* ids) {
    uint64_t base[NBT];
#pragma unroll
    for (int j = 0; j < NBT; ++j) base[j] = (uint64_t)ids[j] * block_bytes + head_bytes;
    // row 0 of the tile in new_k / new_v, as an integer: it wraps below zero
    // when the tile starts before the first new token (only lanes at or past
    // that token load, at addresses inside new_k / new_v)
    const uint64_t nbase = (uint64_t)(((int64_t)(qa - pos0 + kt * kPfKT) * H + h) * RB);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int t = slot_row[r];
      if (t >= kPfKT) continue;
      char* kl = lds + buf * BUF + 16 * NT * r + 1024 * wave;    // this wave's 1 KiB of the round
      char* vl = kl + VOFF;
      const int T = kt * kPfKT + t;          // this thread's key position
      if (APPEND && T >= pos0 && T < n) {
        // a new token: its row of new_k / new_v, same chunk order as in the pools
        load16_to_lds(reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(new_k) + nbase + opaque(noffk[r])), kl);
        load16_to_lds(reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(new_v) + nbase + opaque(noffv[r])), vl);
      } else if (T < n) {
        // the block this thread's row lies in; when a round's rows all lie in
        // one block, that block is known at compile time, and the address is
        // a scalar base plus this lane's offset
        constexpr int RPR = (16 * NT) % RB == 0 ? 16 * NT / RB : 0;    // rows per round, if whole
        const uint64_t b = NBT == 1 ? base[0]
                         : (RPR > 0 && BS % RPR == 0) ? base[(r * RPR / BS) % NBT] : base[(t / BS) % NBT];
        load16_to_lds((const char*)k_cache + b + opaque(offk[r]), kl);
        load16_to_lds((const char*)v_cache + b + opaque(offv[r]), vl);
      } else {
        *reinterpret_cast<u32x4*>(kl + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(vl + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // 8-bit pools: thread i loads bytes 16 i + 16 NT r of the tile (row t, 16
  // elements from e0), into registers, one tile ahead; after the current
  // tile's products it stores them, converted to FMT, as chunks e0 / 8 and
  // e0 / 8 + 1 of row t of the LDS image (swizzled as above).  Rows past n:
  // zero bytes, finite in both formats (E4M3 0, INT8 0 + 128); every query
  // masks them, so their weights are 0.
  const uint64_t head_bytes8 = (uint64_t)h * (BS * D);
  const uint64_t block_bytes8 = (uint64_t)H * (BS * D);
  u32x4 stk[ROUNDS8], stv[ROUNDS8];
  auto stage = [&](int kt, const int64_t* ids) {
#pragma unroll
    for (int r = 0; r < ROUNDS8; ++r) {
      const int P = 16 * (int)threadIdx.x + 16 * NT * r;
      const int t = P / D, e0 = P % D;
      const int T = kt * kPfKT + t;
      stk[r] = stv[r] = u32x4{0u, 0u, 0u, 0u};
      if (P < TB8 && T < n) {
        const uint64_t b = (uint64_t)ids[(t / BS) % NBT] * block_bytes8 + head_bytes8 + (uint64_t)((t % BS) * D + e0);
        stk[r] = load16_cached((const char*)k_cache + b);
        stv[r] = load16_cached((const char*)v_cache + b);
      }
    }
  };
  auto unstage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < ROUNDS8; ++r) {
      const int P = 16 * (int)threadIdx.x + 16 * NT * r;
      if (P >= TB8) continue;
      const int t = P / D, c0 = (P % D) / 8;
      char* kr = lds + buf * BUF + t * RB;
      char* vr = kr + VOFF;
      u32x4 klo, khi, vlo, vhi;
      to_operand<FMT, CFMT>(stk[r], klo, khi);
      to_operand<FMT, CFMT>(stv[r], vlo, vhi);
      *reinterpret_cast<u32x4*>(kr + 16 * (c0 ^ Swz::k(t))) = klo;
      *reinterpret_cast<u32x4*>(kr + 16 * ((c0 + 1) ^ Swz::k(t))) = khi;
      *reinterpret_cast<u32x4*>(vr + 16 * (c0 ^ Swz::v(t))) = vlo;
      *reinterpret_cast<u32x4*>(vr + 16 * ((c0 + 1) ^ Swz::v(t))) = vhi;
    }
  };

  // LDS byte offsets of this lane's operand reads within a tile buffer,
  // fixed for the whole loop.  K: chunk 2c + hb of row col (rows 32 kb + col
  // add 32 kb whole rows).  V^T: column tile dt, row 4 hb + src_k (rows
  // 16 c and 16 c + 8 further add whole rows).  The swizzles depend only on
  // a row's low bits, which those whole-row steps leave alone, so every
  // read is one of these offsets plus a constant.
  const int src_k = (lane & 15) >> 2;        // row offset this lane supplies to a transposing read
  const int src_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // column offset it supplies
  uint32_t koff[D / 16], voff[DP / 32];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) koff[c] = (uint32_t)(col * RB + 16 * ((2 * c + hb) ^ Swz::k(col)));
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) {
    const int d0 = 32 * dt + src_c, t = 4 * hb + src_k;
    voff[dt] = (uint32_t)(VOFF + t * RB + 16 * ((d0 >> 3) ^ Swz::v(t)) + 2 * (d0 & 7));
  }

  auto compute = [&](auto bufc, int kt) {
    constexpr int buf = decltype(bufc)::value;
    const int key0 = kt * kPfKT;
    if (key0 > wave_pos_hi) return;          // every key of the tile is after every query of the wave
    const char* base = lds + buf * BUF;
    f32x16 sacc[KSB];
#pragma unroll
    for (int kb = 0; kb < KSB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int kb = 0; kb < KSB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base + koff[c] + 32 * kb * RB);
        sacc[kb] = Mma<FMT>::mac(a, qop[c], sacc[kb]);
      }
    // causal mask, only where the tile reaches past the wave's first query
    if (key0 + kPfKT - 1 > wave_pos_lo) {
#pragma unroll
      for (int kb = 0; kb < KSB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + 32 * kb + 8 * (e >> 2) + 4 * hb + (e & 3);
          if (key > my_pos) sacc[kb][e] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < KSB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = max_halves(mx);
    const float mt = CFMT == I8 ? __builtin_fmaf(mx, s_mult, -qcorr) : mx * s_mult;
    if (__builtin_amdgcn_ballot_w64(mt > m_slack) != 0) {
      const float m_new = fmaxf(m, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DP / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      m = m_new;
      m_slack = m + kSlack;
      m_ref = ref_of(m);
    }
    u32x4 pb[2 * KSB];
#pragma unroll
    for (int kb = 0; kb < KSB; ++kb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], s_mult, -m_ref));
      }
      // the weights in the operand format; the row sum adds those same
      // rounded weights (v_dot2 with (1, 1)), so numerator and normaliser
      // agree, with half the additions of summing the fp32 values
#pragma unroll
      for (int hc = 0; hc < 2; ++hc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pb[2 * kb + hc][w] = Mma<FMT>::pack(p[8 * hc + 2 * w], p[8 * hc + 2 * w + 1]);
          l = Mma<FMT>::sum2(pb[2 * kb + hc][w], l);
        }
    }
    // V^T operand of 16-key chunk c: rows 16c + 4hb + {0..3} and 16c + 8 + 4hb + {0..3}
    // of column 32 dt + col, two transposing reads (see above)
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
#pragma unroll
      for (int c = 0; c < 2 * KSB; ++c) {
        const char* a_lo = base + voff[dt] + 16 * c * RB;
        const char* a_hi = a_lo + 8 * RB;
        const u32x2 lw = lds_read_tr16x4(a_lo), hw = lds_read_tr16x4(a_hi);
        o[dt] = Mma<FMT>::mac(u32x4{lw.x, lw.y, hw.x, hw.y}, pb[c], o[dt]);
      }
    }
  };

  // APPEND: new tokens [max(i_base, 0), i_end) of head h go to their slots,
  // exactly as the cache write stores them (a bit copy: the pools hold the q
  // format).  Those tokens are the last keys of this workgroup's range, so
  // each of their rows passes through an LDS tile (read from new_k / new_v,
  // see fetch); it is stored to the pools from there, while the tile is
  // resident, instead of being loaded from global memory a second time.  No
  // workgroup reads them back from the pools, so the result is that of the
  // cache write followed by the prompt attention.
  const int store_lo = pos0 + max(i_base, 0);    // positions [store_lo, kv_end) are stored here
  // the byte offset of each of those rows in the pools (-1: not stored), from
  // its slot, found once before the loop (visible after the loop's first barrier)
  __shared__ int64_t new_dst[APPEND ? kPfQT : 1];
  if constexpr (APPEND) {
    if (threadIdx.x < kPfQT) {
      const int i = i_base + (int)threadIdx.x;
      const int slot = i >= 0 ? slot_mapping[qa + i] : -1;
      new_dst[threadIdx.x] = (slot < 0 || slot / BS >= NB) ? (int64_t)-1
                           : (int64_t)(tile_base<D, BS>(slot / BS, h, H) * EB + (size_t)(slot % BS) * RB);
    }
  }
  auto store_new_rows = [&](auto bufc, int kt) {
    constexpr int buf = decltype(bufc)::value;
    constexpr int CPR = RB / 16;             // 16-byte chunks per row
    const int key0 = kt * kPfKT;
    const int lo = max(key0, store_lo), hi = min(key0 + kPfKT, kv_end);
    if (lo >= hi) return;
    const char* kt_lds = lds + buf * BUF;
    for (int c = threadIdx.x; c < (hi - lo) * CPR; c += NT) {
      const int T = lo + c / CPR, ch = c % CPR, t = T - key0;
      const int64_t row_dst = new_dst[T - pos0 - i_base];
      if (row_dst < 0) continue;             // padding and out-of-pool slots are skipped
      const u32x4 kw = *reinterpret_cast<const u32x4*>(kt_lds + t * RB + 16 * (ch ^ Swz::k(t)));
      const u32x4 vw = *reinterpret_cast<const u32x4*>(kt_lds + VOFF + t * RB + 16 * (ch ^ Swz::v(t)));
      const size_t dst = (size_t)row_dst + 16 * ch;
      __builtin_nontemporal_store(kw, reinterpret_cast<u32x4*>((char*)const_cast<void*>(k_cache) + dst));
      __builtin_nontemporal_store(vw, reinterpret_cast<u32x4*>((char*)const_cast<void*>(v_cache) + dst));
    }
  };

  int64_t ids_next[NBT];
  {
    int64_t ids0[NBT];
    tile_ids(0, ids0);
    if constexpr (DIRECT) {
      fetch(0, 0, ids0);
    } else {
      stage(0, ids0);
      unstage(0);
    }
    tile_ids(1, ids_next);
  }
  __builtin_amdgcn_s_waitcnt(0);             // the direct loads (and zero stores) have landed in LDS
  __syncthreads();
  // The loop runs two tiles per pass, one per buffer, so that the buffer is
  // a compile-time constant: its offset and the whole-row steps above then
  // go into the LDS reads' immediate offsets, and each read needs no address
  // arithmetic (about 20 vector instructions less per tile and wave).
  auto step = [&](auto bufc, int kt) {
    constexpr int buf = decltype(bufc)::value;
    // before the products, so that the stores retire meanwhile
    if constexpr (APPEND) store_new_rows(bufc, kt);
    if (kt + 1 < nkt) {
      // into the buffer last read in the previous step
      if constexpr (DIRECT) fetch(kt + 1, buf ^ 1, ids_next);
      else stage(kt + 1, ids_next);
      tile_ids(kt + 2, ids_next);
    }
    compute(bufc, kt);
    if constexpr (!DIRECT) {
      if (kt + 1 < nkt) unstage(buf ^ 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nkt) step(std::integral_constant<int, 1>{}, kt + 1);
  }

  if (!q_ok) return;
  const float lt = sum_halves(l);
  const float inv = out_mult / lt;           // the query's own key is visible, so lt > 0
  if constexpr (CFMT == I8) {
    // every value element carried + 128: O holds 128 * (sum of the rounded
    // weights) = 128 * lt too much
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] = __builtin_fmaf(-Chunk<I8>::offset, lt, o[dt][e]);
  }
  char* orow = (char*)out + ((size_t)(qa + my_q) * H + h) * D * EB;
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * dt + 8 * j + 4 * hb;
      if (DP != D && d0 >= D) continue;        // padding rows
      const uint32_t w0 = Mma<FMT>::pack(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv);
      const uint32_t w1 = Mma<FMT>::pack(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d0 * EB) = u32x2{w0, w1};
    }
}

template <int FMT, int CFMT, int D, int BS>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int tiles = (a.max_q_len + kPfQT - 1) / kPfQT;
  dim3 grid(a.H, tiles, a.S);
  if constexpr (CFMT == FMT) {
    if (a.slot_mapping) {
      hipLaunchKernelGGL((paged_prefill_kernel<FMT, CFMT, D, BS, true>), grid, dim3(kPfWaves * 64), 0, st, a.out,
                         a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.cu_q_lens, a.Tq, a.H, a.MB,
                         a.NB, a.s_mult, 1.0f, nullptr, nullptr, a.new_k, a.new_v, a.slot_mapping);
      return hipGetLastError();
    }
  } else if (a.slot_mapping) {
    // 8-bit pools: the cache write quantises the new tokens first (doing it
    // in the prompt kernel would cost registers), then the plain kernel reads
    // them back from the pools like the cached context
    const hipError_t e = launch_reshape_and_cache(a.new_k, a.new_v, const_cast<void*>(a.k_cache),
                                                  const_cast<void*>(a.v_cache), a.slot_mapping, a.Tq, a.H, D, BS,
                                                  a.NB, FMT, CFMT, a.k_scale, a.v_scale, a.k_scales, a.v_scales, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((paged_prefill_kernel<FMT, CFMT, D, BS, false>), grid, dim3(kPfWaves * 64), 0, st, a.out, a.q,
                     a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.cu_q_lens, a.Tq, a.H, a.MB, a.NB,
                     a.s_mult, a.out_mult, a.k_scales, a.v_scales, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

template <int FMT, int CFMT, int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t st) {
  return a.BS == 16 ? launch_prefill_t<FMT, CFMT, D, 16>(a, st) : launch_prefill_t<FMT, CFMT, D, 32>(a, st);
}

template <int FMT, int CFMT>
static hipError_t launch_prefill_fmt(const PrefillArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_prefill_d<FMT, CFMT, 64>(a, st);
    case 80: return launch_prefill_d<FMT, CFMT, 80>(a, st);
    case 96: return launch_prefill_d<FMT, CFMT, 96>(a, st);
    case 128: return launch_prefill_d<FMT, CFMT, 128>(a, st);
    case 256: return launch_prefill_d<FMT, CFMT, 256>(a, st);       // one workgroup per CU (254 VGPRs)
  }
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_prefill_cache(const PrefillArgs& a, hipStream_t st) {
  if (a.c_fmt == FMT) return launch_prefill_fmt<FMT, FMT>(a, st);
  if (a.c_fmt == E4M3) return launch_prefill_fmt<FMT, E4M3>(a, st);
  if (a.c_fmt == I8) return launch_prefill_fmt<FMT, I8>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.max_q_len <= 0) return hipSuccess;
  if (a.fmt == BF16) return launch_prefill_cache<BF16>(a, st);
  if (a.fmt == F16) return launch_prefill_cache<F16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace pkv

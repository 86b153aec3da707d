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
// queries.  Keys are consumed in tiles of 32 tokens, staged through LDS
// (double-buffered, one barrier per tile): K row-major [token][d] and V
// transposed [d][token], so that both MFMA operands read contiguously along
// their contraction index.
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
// consistently on both sides.

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
};
template <> struct Mma<F16> {
  __device__ __forceinline__ static f32x16 mac(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2));
  }
};

// Tunables (compile-time): keys per tile (a multiple of 32), LDS buffers
// per tile stage (2: one barrier per tile; 1: two), and the workgroups per
// CU the register budget is sized for.
#ifndef PKV_PF_KT
#define PKV_PF_KT 32
#endif
#ifndef PKV_PF_NBUF
#define PKV_PF_NBUF 2
#endif
#ifndef PKV_PF_MINWG
#define PKV_PF_MINWG 3
#endif

constexpr int kPfWaves = 4;                  // waves per workgroup
constexpr int kPfQW = 32;                    // queries per wave
constexpr int kPfQT = kPfWaves * kPfQW;      // queries per workgroup
constexpr int kPfKT = PKV_PF_KT;             // keys per tile
constexpr int kPfBufs = PKV_PF_NBUF;
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

#ifndef PKV_PF_SETPRIO
#define PKV_PF_SETPRIO 0
#endif

template <int FMT, int D, int BS>
__global__ __launch_bounds__(kPfWaves * 64, D >= 256 ? 1 : PKV_PF_MINWG) void paged_prefill_kernel(
    void* __restrict__ out, const void* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens, int Tq, int H, int MB,
    int NB, float s_mult) {
  constexpr int EB = 2;
  constexpr int DC = D / 8;                  // 16-byte chunks per token row
  constexpr int DP = (D + 31) / 32 * 32;     // rows of O^T: D rounded up to whole 32-row MFMA tiles
  constexpr int KROW = D * EB + 16;          // LDS bytes per K row (padding keeps b128 reads conflict-free)
  constexpr int VROW = kPfKT * EB + 8;       // LDS bytes per V^T row (padding keeps b64 reads conflict-free)
  constexpr int KBUF = kPfKT * KROW;
  constexpr int BUF = KBUF + DP * VROW;      // V^T rows D .. DP-1 stay zero
  // A thread moves pairs of key rows (2tp, 2tp + 1) of one 16-byte column
  // chunk dc: NPAIR pairs per tile, PPT per thread (the last ones may be idle).
  constexpr int NPAIR = (kPfKT / 2) * DC;
  constexpr int PPT = (NPAIR + kPfWaves * 64 - 1) / (kPfWaves * 64);
  constexpr int CPT = 2 * PPT;               // 16-byte chunks per thread per tile, K and V each
  static_assert(D % 16 == 0, "head size must be a multiple of 16");
  constexpr int KSB = kPfKT / 32;            // 32-key blocks of S^T per tile
  static_assert(kPfKT % 32 == 0 && kPfKT % BS == 0, "tile must be whole 32-key blocks and whole cache blocks");
  __shared__ __attribute__((aligned(16))) char lds[kPfBufs * BUF];

  const int h = blockIdx.x;
  const int tile = blockIdx.y;
  const int s = blockIdx.z;
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
  const int wave_pos_hi = pos0 + wq0 + kPfQW - 1;
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

  f32x16 o[DP / 32];
#pragma unroll
  for (int i = 0; i < DP / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m = -INFINITY;                       // reference for the exponentials (log2 units)
  float l = 0.0f;                            // this lane's part of the running sum

  // Physical block ids of one key tile: NBT uniform values, read with scalar
  // loads one tile before the K/V loads that use them.  Ids past the
  // sequence are never read from the table; ids outside the pool read block 0.
  constexpr int NBT = kPfKT / BS;
  auto tile_ids = [&](int kt, int64_t* ids) {
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
      const int lb = __builtin_amdgcn_readfirstlane(kt * NBT + j);
      int64_t b = lb < nblocks ? (int64_t)table[lb] : 0;
      if ((uint64_t)b >= (uint64_t)NB) b = 0;
      ids[j] = b;
    }
  };

  // Which 16-byte chunk of the key tile a thread moves, for r < CPT: rows
  // 2tp and 2tp + 1 of column chunk dc for pair id = thread + 256 * (r / 2),
  // so that it can write V^T as pairs of keys (one 32-bit LDS store per
  // element of the chunk, consecutive lanes on consecutive banks).  A thread
  // whose pair id is past NPAIR has nothing to move.
  auto chunk_of = [&](int r, int& t, int& dc) -> bool {
    const int id = threadIdx.x + (r >> 1) * kPfWaves * 64;
    t = 2 * (id % (kPfKT / 2)) + (r & 1);
    dc = id / (kPfKT / 2);
    return NPAIR % (kPfWaves * 64) == 0 || id < NPAIR;
  };

  // global -> registers for one key tile (rows past n are zero)
  u32x4 kr[CPT], vr[CPT];
  auto fetch = [&](int kt, const int64_t* ids) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      int t, dc;
      const bool mine = chunk_of(r, t, dc);
      const int tok = kt * kPfKT + t;
      if (mine && tok < n) {
        const int64_t b = NBT == 1 ? ids[0] : ids[(t / BS) % NBT];
        const size_t off = (tile_base<D, BS>(b, h, H) + (size_t)(tok % BS) * D + 8 * dc) * EB;
        kr[r] = load16_cached((const char*)k_cache + off);
        vr[r] = load16_cached((const char*)v_cache + off);
      } else {
        kr[r] = u32x4{0u, 0u, 0u, 0u};
        vr[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // registers -> LDS buffer: K as rows, V transposed
  auto stage = [&](int buf) {
    char* base = lds + buf * BUF;
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      int t, dc;
      if (!chunk_of(r, t, dc)) continue;
      *reinterpret_cast<u32x4*>(base + t * KROW + dc * 16) = kr[r];
      if (r & 1) {                           // rows t - 1 (chunk r - 1) and t: one 32-bit pair per element
        char* vt = base + KBUF + (8 * dc) * VROW + (t - 1) * EB;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a = vr[r - 1][w], b = vr[r][w];
          // (low halves of a, b) and (high halves of a, b)
          *reinterpret_cast<uint32_t*>(vt + (2 * w) * VROW) = __builtin_amdgcn_perm(b, a, 0x05040100u);
          *reinterpret_cast<uint32_t*>(vt + (2 * w + 1) * VROW) = __builtin_amdgcn_perm(b, a, 0x07060302u);
        }
      }
    }
  };

  auto compute = [&](int buf, int kt) {
    const int key0 = kt * kPfKT;
    if (key0 > wave_pos_hi) return;          // every key of the tile is after every query of the wave
    const char* base = lds + buf * BUF;
    f32x16 sacc[KSB];
#pragma unroll
    for (int kb = 0; kb < KSB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
    if (PKV_PF_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int kb = 0; kb < KSB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base + (32 * kb + col) * KROW + (16 * c + 8 * hb) * EB);
        sacc[kb] = Mma<FMT>::mac(a, qop[c], sacc[kb]);
      }
    if (PKV_PF_SETPRIO) __builtin_amdgcn_s_setprio(0);
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
    const float mt = mx * s_mult;            // the tile's largest scaled score for this query
    // The reference m only has to keep every weight 2^(z - m) <= 2^kSlack: a
    // larger maximum in this tile moves it (and rescales O and l by the
    // same factor) only when it exceeds m by more than kSlack for some
    // query of the wave.  The final O / l does not depend on m.
    if (__builtin_amdgcn_ballot_w64(mt > m + kSlack) != 0) {
      const float m_new = fmaxf(m, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DP / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      m = m_new;
    }
    const float m_ref = (m == -INFINITY) ? 0.0f : m;
    // P^T as B operands, one per 16-key chunk c (keys 16c + 4hb + {0..3},
    // 16c + 8 + 4hb + {0..3} of the tile)
    u32x4 pb[2 * KSB];
#pragma unroll
    for (int kb = 0; kb < KSB; ++kb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], s_mult, -m_ref));
        l += p[e];
      }
#pragma unroll
      for (int hc = 0; hc < 2; ++hc)
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[2 * kb + hc][w] = Mma<FMT>::pack(p[8 * hc + 2 * w], p[8 * hc + 2 * w + 1]);
    }
    if (PKV_PF_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
      const char* vrow = base + KBUF + (32 * dt + col) * VROW;
#pragma unroll
      for (int c = 0; c < 2 * KSB; ++c) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (16 * c + 4 * hb) * EB);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (16 * c + 8 + 4 * hb) * EB);
        o[dt] = Mma<FMT>::mac(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[c], o[dt]);
      }
    }
    if (PKV_PF_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };

  if constexpr (DP != D) {
    // the padding rows of V^T in both buffers: zero once, never written again
    for (int i = threadIdx.x; i < kPfBufs * (DP - D) * (VROW / 4); i += kPfWaves * 64) {
      const int b = i / ((DP - D) * (VROW / 4)), r = i % ((DP - D) * (VROW / 4));
      *reinterpret_cast<uint32_t*>(lds + b * BUF + KBUF + D * VROW + 4 * r) = 0u;
    }
  }

  int64_t ids_next[NBT];
  {
    int64_t ids0[NBT];
    tile_ids(0, ids0);
    fetch(0, ids0);
    tile_ids(1, ids_next);
  }
  stage(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      fetch(kt + 1, ids_next);
      tile_ids(kt + 2, ids_next);
    }
    if constexpr (kPfBufs == 2) {
      compute(kt & 1, kt);
      if (more) stage((kt + 1) & 1);
    } else {
      compute(0, kt);
      if (more) {
        __syncthreads();                     // every wave is done reading the buffer
        stage(0);
      }
    }
    __syncthreads();
  }

  if (!q_ok) return;
  const float lt = sum_halves(l);
  const float inv = 1.0f / lt;               // the query's own key is visible, so lt > 0
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

template <int FMT, int D, int BS>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int tiles = (a.max_q_len + kPfQT - 1) / kPfQT;
  dim3 grid(a.H, tiles, a.S);
  hipLaunchKernelGGL((paged_prefill_kernel<FMT, D, BS>), grid, dim3(kPfWaves * 64), 0, st, a.out, a.q, a.k_cache,
                     a.v_cache, a.block_tables, a.context_lens, a.cu_q_lens, a.Tq, a.H, a.MB, a.NB, a.s_mult);
  return hipGetLastError();
}

template <int FMT, int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t st) {
  return a.BS == 16 ? launch_prefill_t<FMT, D, 16>(a, st) : launch_prefill_t<FMT, D, 32>(a, st);
}

template <int FMT>
static hipError_t launch_prefill_fmt(const PrefillArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_prefill_d<FMT, 64>(a, st);
    case 80: return launch_prefill_d<FMT, 80>(a, st);
    case 96: return launch_prefill_d<FMT, 96>(a, st);
    case 128: return launch_prefill_d<FMT, 128>(a, st);
    case 256: return launch_prefill_d<FMT, 256>(a, st);       // one workgroup per CU (254 VGPRs)
  }
  return hipErrorInvalidValue;
}

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.max_q_len <= 0) return hipSuccess;
  if (a.fmt == BF16) return launch_prefill_fmt<BF16>(a, st);
  if (a.fmt == F16) return launch_prefill_fmt<F16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace pkv

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

constexpr int kPfWaves = 4;                  // waves per workgroup
constexpr int kPfQW = 32;                    // queries per wave
constexpr int kPfQT = kPfWaves * kPfQW;      // queries per workgroup
constexpr int kPfKT = 32;                    // keys per tile

__device__ __forceinline__ u32x4 load16_cached(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int FMT, int D, int BS>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_kernel(
    void* __restrict__ out, const void* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens, int Tq, int H, int MB,
    int NB, float s_mult) {
  constexpr int EB = 2;
  constexpr int DC = D / 8;                  // 16-byte chunks per token row
  constexpr int KROW = D * EB + 16;          // LDS bytes per K row (padding keeps b128 reads conflict-free)
  constexpr int VROW = kPfKT * EB + 8;       // LDS bytes per V^T row (padding keeps b64 reads conflict-free)
  constexpr int KBUF = kPfKT * KROW;
  constexpr int BUF = KBUF + D * VROW;
  constexpr int CPT = kPfKT * DC / (kPfWaves * 64);   // 16-byte chunks per thread per tile, K and V each
  static_assert(CPT >= 1 && kPfKT * DC % (kPfWaves * 64) == 0, "tile does not split over the threads");
  static_assert(kPfKT % BS == 0 || BS % kPfKT == 0, "tile and block sizes must nest");
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

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

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m = -INFINITY;                       // running max of the scaled scores (log2 units)
  float l = 0.0f;                            // this lane's part of the running sum

  // global -> registers for one key tile (rows past n are zero)
  u32x4 kr[CPT], vr[CPT];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int ci = threadIdx.x + r * kPfWaves * 64;
      const int t = ci / DC, dc = ci % DC;
      const int tok = kt * kPfKT + t;
      if (tok < n) {
        int64_t b = table[tok / BS];
        if ((uint64_t)b >= (uint64_t)NB) b = 0;      // out-of-range id: stay inside the pool
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
      const int ci = threadIdx.x + r * kPfWaves * 64;
      const int t = ci / DC, dc = ci % DC;
      *reinterpret_cast<u32x4*>(base + t * KROW + dc * 16) = kr[r];
      char* vt = base + KBUF + (8 * dc) * VROW + t * EB;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(vt + e * VROW) = (uint16_t)(vr[r][e >> 1] >> (16 * (e & 1)));
    }
  };

  auto compute = [&](int buf, int kt) {
    const int key0 = kt * kPfKT;
    if (key0 > wave_pos_hi) return;          // every key of the tile is after every query of the wave
    const char* base = lds + buf * BUF;
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(base + col * KROW + (16 * c + 8 * hb) * EB);
      sacc = Mma<FMT>::mac(a, qop[c], sacc);
    }
    // causal mask, only where the tile reaches past the wave's first query
    if (key0 + kPfKT - 1 > wave_pos_lo) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + 8 * (e >> 2) + 4 * hb + (e & 3);
        if (key > my_pos) sacc[e] = -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * s_mult);
    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
    m = m_new;
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], s_mult, -m_ref));
      l += p[e];
    }
    u32x4 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) pb[c][w] = Mma<FMT>::pack(p[8 * c + 2 * w], p[8 * c + 2 * w + 1]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* vrow = base + KBUF + (32 * dt + col) * VROW;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (16 * c + 4 * hb) * EB);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (16 * c + 8 + 4 * hb) * EB);
        o[dt] = Mma<FMT>::mac(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[c], o[dt]);
      }
    }
  };

  fetch(0);
  stage(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) fetch(kt + 1);
    compute(kt & 1, kt);
    if (more) stage((kt + 1) & 1);
    __syncthreads();
  }

  if (!q_ok) return;
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;               // the query's own key is visible, so lt >= 1
  char* orow = (char*)out + ((size_t)(qa + my_q) * H + h) * D * EB;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * dt + 8 * j + 4 * hb;
      uint32_t w0, w1;
      if constexpr (FMT == BF16) {
        w0 = f32_to_bf16_rn(o[dt][4 * j] * inv) | ((uint32_t)f32_to_bf16_rn(o[dt][4 * j + 1] * inv) << 16);
        w1 = f32_to_bf16_rn(o[dt][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16_rn(o[dt][4 * j + 3] * inv) << 16);
      } else {
        w0 = f32_to_f16_rn(o[dt][4 * j] * inv) | ((uint32_t)f32_to_f16_rn(o[dt][4 * j + 1] * inv) << 16);
        w1 = f32_to_f16_rn(o[dt][4 * j + 2] * inv) | ((uint32_t)f32_to_f16_rn(o[dt][4 * j + 3] * inv) << 16);
      }
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

template <int FMT>
static hipError_t launch_prefill_fmt(const PrefillArgs& a, hipStream_t st) {
  if (a.D == 64) return a.BS == 16 ? launch_prefill_t<FMT, 64, 16>(a, st) : launch_prefill_t<FMT, 64, 32>(a, st);
  return a.BS == 16 ? launch_prefill_t<FMT, 128, 16>(a, st) : launch_prefill_t<FMT, 128, 32>(a, st);
}

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.max_q_len <= 0) return hipSuccess;
  if (a.fmt == BF16) return launch_prefill_fmt<BF16>(a, st);
  if (a.fmt == F16) return launch_prefill_fmt<F16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace pkv

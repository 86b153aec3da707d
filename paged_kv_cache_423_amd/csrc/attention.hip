// Paged-attention decode for gfx950: one query token per (sequence, head)
// attends over K/V held in fixed-size physical blocks reached through the
// sequence's block table ("vLLM-v0.17.1技术解析：PagedAttention内存管理与显存
// 优化技巧" §2.2; "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战" §2.1).
//
// Work split.  The context of each sequence is cut into partitions of
// PART_BLOCKS physical blocks.  One workgroup of NW wave64s handles one
// (partition, head, sequence); wave w takes the partition's blocks
// w, w + NW, ...  Within a wave, one 16-byte load per lane covers RPL
// consecutive token rows of one (block, head) tile, so each wave-wide load
// reads 1 KiB of contiguous HBM.  A lane owns a fixed slice of EPL head
// elements of rows rg, rg + RPL, ... of every block it visits.
//
// Softmax.  Each lane keeps an online max / sum / weighted-V state for its
// row group (base-2 exponent, log2(e) folded into the q scale).  Row dot
// products are summed across the LPR lanes of a row with DPP; no other
// cross-lane traffic happens inside the block loop.  At the end of a
// partition, the row groups of a wave and then the waves of the workgroup
// are merged with the usual rescaling.  A sequence that fits in one
// partition writes its output directly; otherwise the partition writes
// (max, sum, weighted V) to the workspace and a second kernel merges the
// partitions.  The order of arithmetic depends only on logical token
// positions, never on physical block ids.
//
// This is a matrix-vector path (about 1 flop per byte of K/V at 16-bit), so
// HBM bandwidth bounds it and it uses no MFMA.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

// Every rounding in this file is the one written: no multiply-add is fused
// unless it is written as fmaf.  The per-sequence and the grouped decode
// then round identically whatever the surrounding control flow, which keeps
// their results bitwise equal.
#pragma clang fp contract(off)

namespace pkv {

template <int CFMT, int D>
struct Tile {
  static constexpr int EB = FmtInfo<CFMT>::bytes;
  static constexpr int EPL = 16 / EB;          // elements per lane per 16-B load
  static constexpr int ACT = D / EPL;          // lanes that hold part of a token row
  // lanes per token row: ACT rounded up to a power of two; the lanes past
  // ACT load nothing and add zeros (head sizes such as 80 and 96)
  static constexpr int LPR = ACT <= 1 ? 1 : ACT <= 2 ? 2 : ACT <= 4 ? 4 : ACT <= 8 ? 8
                           : ACT <= 16 ? 16 : ACT <= 32 ? 32 : 64;
  static constexpr int RPL = 64 / LPR;         // rows per wave-wide load
  static_assert(D % EPL == 0 && ACT >= 1 && ACT <= 64, "bad tile");
};

// APPEND: the step's new tokens are written into the pools by this kernel
// (see below) instead of by a separate cache write before it.
template <int QFMT, int CFMT, int D, int BS, int NW, int PART_BLOCKS, bool APPEND>
__global__ __launch_bounds__(NW * 64) void paged_decode_kernel(
    void* __restrict__ out, const void* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int H, int MB, int NB, float q_mult, float out_mult,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, int max_parts, const void* __restrict__ new_k, const void* __restrict__ new_v,
    const int32_t* __restrict__ slot_mapping) {
  using T = Tile<CFMT, D>;
  constexpr int EPL = T::EPL, LPR = T::LPR, RPL = T::RPL, EB = T::EB, ACT = T::ACT;
  constexpr int LPB = BS / RPL;                // loads per lane per block tile
  // A block tile is consumed in SUB sub-tiles of LPS loads per lane (at most
  // 4 for K and 4 for V per register stage), rows sub * RPL * LPS onwards.
  constexpr int LPS = LPB < 4 ? LPB : 4;
  constexpr int SUB = LPB / LPS;
  constexpr int MAXB = PART_BLOCKS / NW;       // blocks per wave per partition
  static_assert(BS % RPL == 0 && LPB % LPS == 0, "block size must be a multiple of rows per load");
  static_assert(PART_BLOCKS % NW == 0, "partition must split evenly over the waves");

  const int h = blockIdx.x;
  const int p = blockIdx.y;
  const int s = blockIdx.z;
  // 8-bit pools with one scale per head: this head's scales multiply the q
  // scale and the output, exactly as the pool's one scale does otherwise
  if constexpr (scaled_format(CFMT)) {
    if (k_scales) q_mult *= k_scales[h];
    if (v_scales) out_mult *= v_scales[h];
  }
  const int lane = threadIdx.x & 63;
  // wave index as a scalar, so that block-table reads are scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = lane / LPR;                   // row group
  const int col = lane % LPR;                  // column lane
  const bool col_ok = ACT == LPR || col < ACT; // this lane holds part of the row

  // The wave's first block id depends only on its place in the grid, so it
  // is read at once, beside the length: the first K/V loads then wait for
  // one table read rather than for the length and then the table.
  const int32_t* table = block_tables + (size_t)s * MB;
  const int first_id_pos = p * PART_BLOCKS + wave;
  const int32_t first_id = first_id_pos < MB ? table[first_id_pos] : 0;

  // lengths outside [0, MB*BS] are clamped so that no access leaves the
  // table, the pools or the workspace
  const int n = min(max(context_lens[s], 0), MB * BS);
  const int nblocks = (n + BS - 1) / BS;
  const int nparts = (nblocks + PART_BLOCKS - 1) / PART_BLOCKS;
  const size_t out_base = ((size_t)s * H + h) * D;

  // APPEND (pools whose cache write is a bit copy): this head's row of the
  // sequence's new token goes to slot_mapping[s], the slot of position
  // n - 1, exactly as the cache write stores it.  Only the wave that reads
  // the sequence's last block reads that position, so that wave does the
  // write, and never reads the row back: each of its lanes loads the new
  // row's chunk of its own columns up front, uses it in place of what it
  // loads for position n - 1 (the same bytes the write stores, so the same
  // arithmetic), and stores it after its block loop.  With n = 0 nothing
  // reads the slot and wave 0 of partition 0 writes it.  The same workgroup
  // never reads the row from memory, so no ordering between its lanes or
  // waves is needed; another sequence never reads it (copy-on-write).
  static_assert(!APPEND || QFMT == CFMT, "the appending decode stores the new rows bit for bit");
  int wslot = -1;                              // >= 0: this wave writes the row at that slot
  u32x4 new_kc = {0u, 0u, 0u, 0u}, new_vc = {0u, 0u, 0u, 0u};   // the new row's chunk of this lane's columns
  if constexpr (APPEND) {
    const bool writer = nparts > 0 ? (p == nparts - 1 && wave == (nblocks - 1 - p * PART_BLOCKS) % NW)
                                   : (p == 0 && wave == 0);
    if (writer) {
      const int slot = slot_mapping[s];
      if (slot >= 0 && slot / BS < NB) {       // padding and out-of-pool slots are skipped
        wslot = slot;
        if (col_ok) {
          const size_t src = (out_base + (size_t)col * EPL) * EB;
          new_kc = load16((const char*)new_k + src);
          new_vc = load16((const char*)new_v + src);
        }
      }
    }
  }
  auto append_store = [&]() {
    if (APPEND && wslot >= 0 && rg == 0 && col_ok) {
      const size_t dst = (tile_base<D, BS>(wslot / BS, h, H) + (size_t)(wslot % BS) * D + (size_t)col * EPL) * EB;
      // non-temporal: nothing in this kernel reads the row back, and plain
      // stores cost the long-context decode about 1% more
      __builtin_nontemporal_store(new_kc, reinterpret_cast<u32x4*>((char*)const_cast<void*>(k_cache) + dst));
      __builtin_nontemporal_store(new_vc, reinterpret_cast<u32x4*>((char*)const_cast<void*>(v_cache) + dst));
    }
  };

  if (p >= nparts) {
    // n = 0: the output is defined as zeros
    append_store();
    if (p == 0)
      for (int d = threadIdx.x; d < D; d += NW * 64) store_elem<QFMT>(out, out_base + d, 0.0f);
    return;
  }

  const int blk_begin = p * PART_BLOCKS;
  const int blk_end = min(blk_begin + PART_BLOCKS, nblocks);
  const int full_end = min(blk_end, n / BS);   // blocks with every row < n
  const int first = blk_begin + wave;          // this wave takes first, first + NW, ...
  const int nb = first < blk_end ? (blk_end - first + NW - 1) / NW : 0;

  // this wave's physical block ids, read up front (uniform, scalar loads)
  int64_t ids[MAXB];
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    int64_t b = i < nb ? (int64_t)(i == 0 ? first_id : table[first + i * NW]) : 0;
    if ((uint64_t)b >= (uint64_t)NB) b = 0;    // out-of-range id: stay inside the pool
    ids[i] = b;
  }

  // this lane's q slice, pre-multiplied by scale * log2(e) (* k_scale)
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = col_ok ? load_elem<QFMT>(q, out_base + col * EPL + e) * q_mult : 0.0f;
  // INT8 keys are read as byte + 128: the lane's dot products then carry
  // 128 * (sum of its q slice) too much, taken off once per row
  float qoff = 0.0f;
  if constexpr (CFMT == I8) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qoff += qv[e];
    qoff *= -Chunk<I8>::offset;
  }

  const char* kbase = (const char*)k_cache;
  const char* vbase = (const char*)v_cache;
  const size_t lane_off = ((size_t)rg * D + (size_t)col * EPL) * EB;

  float m = -INFINITY, l = 0.0f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

  // two register stages: the loads of unit u + 1 (a sub-tile of a block)
  // are in flight while unit u is being reduced
  u32x4 kc[2][LPS], vc[2][LPS];
  auto issue = [&](int stage, int64_t phys, int sub) {
    const size_t tb = tile_base<D, BS>(phys, h, H) * EB + lane_off + (size_t)sub * LPS * RPL * D * EB;
#pragma unroll
    for (int i = 0; i < LPS; ++i)
      kc[stage][i] = col_ok ? load16(kbase + tb + (size_t)i * RPL * D * EB) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < LPS; ++i)
      vc[stage][i] = col_ok ? load16(vbase + tb + (size_t)i * RPL * D * EB) : u32x4{0u, 0u, 0u, 0u};
  };
  auto consume = [&](int stage, int j, int sub) {
    if (APPEND && wslot >= 0 && j == nblocks - 1) {   // wave-uniform: the writer's last block
      const int t0 = j * BS + sub * LPS * RPL + rg;
#pragma unroll
      for (int i = 0; i < LPS; ++i) {
        if (t0 + i * RPL == n - 1) {           // the new token's row: the values the write stores
          kc[stage][i] = new_kc;
          vc[stage][i] = new_vc;
        }
      }
    }
    float z[LPS];
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      float kf[EPL];
      Chunk<CFMT>::to_f32(kc[stage][i], kf);
      float dot = qoff;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[e], kf[e], dot);
      z[i] = group_sum<LPR>(dot);
    }
    if (j >= full_end) {                       // wave-uniform: the sequence's last block
      const int t0 = j * BS + sub * LPS * RPL + rg;
#pragma unroll
      for (int i = 0; i < LPS; ++i) {
        if (t0 + i * RPL >= n) {
          z[i] = -INFINITY;
          vc[stage][i] = u32x4{0u, 0u, 0u, 0u};   // rows past n may hold anything
        }
      }
    }
    float zmax = z[0];
#pragma unroll
    for (int i = 1; i < LPS; ++i) zmax = fmaxf(zmax, z[i]);
    const float m_new = fmaxf(m, zmax);
    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const float pi = __builtin_amdgcn_exp2f(z[i] - m_ref);
      l += pi;
      float vf[EPL];
      Chunk<CFMT>::to_f32(vc[stage][i], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(pi, vf[e], acc[e]);
    }
    m = m_new;
  };

  // units u = i * SUB + sub: block i of this wave, sub-tile sub
  const int nunits = nb * SUB;
  if (nunits > 0) issue(0, ids[0], 0);
#pragma unroll
  for (int u = 0; u < MAXB * SUB; ++u) {
    if (u < nunits) {
      if (u + 1 < nunits) issue((u + 1) & 1, ids[(u + 1) / SUB], (u + 1) % SUB);
      consume(u & 1, first + (u / SUB) * NW, u % SUB);
    }
  }
  append_store();

  // merge the RPL row groups of this wave (lanes col, col + LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float m_o = __shfl_xor(m, off);
    const float l_o = __shfl_xor(l, off);
    const float m_new = fmaxf(m, m_o);
    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float a = __builtin_amdgcn_exp2f(m - m_ref), b = __builtin_amdgcn_exp2f(m_o - m_ref);
    l = __builtin_fmaf(l, a, l_o * b);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float acc_o = __shfl_xor(acc[e], off);
      acc[e] = __builtin_fmaf(acc[e], a, acc_o * b);
    }
    m = m_new;
  }

  // merge the NW waves through LDS
  __shared__ float s_acc[NW][D];
  __shared__ float s_m[NW], s_l[NW];
  if (lane < ACT) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wave][lane * EPL + e] = acc[e];
  }
  if (lane == 0) { s_m[wave] = m; s_l[wave] = l; }
  __syncthreads();

  for (int d = threadIdx.x; d < D; d += NW * 64) {
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w]);
    // a processed partition holds at least one token, so M is finite
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w] - M);
      L = __builtin_fmaf(s_l[w], f, L);
      A = __builtin_fmaf(s_acc[w][d], f, A);
    }
    // INT8 values were summed as byte + 128: A holds 128 * L too much
    if constexpr (CFMT == I8) A = __builtin_fmaf(-Chunk<I8>::offset, L, A);
    if (nparts == 1) {
      store_elem<QFMT>(out, out_base + d, (A / L) * out_mult);
    } else {
      const size_t part = ((size_t)s * H + h) * max_parts + p;
      ws_acc[part * D + d] = A;
      if (d == 0) { ws_ml[2 * part] = M; ws_ml[2 * part + 1] = L; }
    }
  }
}

// Shared-prefix decode ("在A10G上榨干LLaMA-7B" §2.2: sequences forked from
// one prompt map the same physical blocks for it, which is stored once).
// One workgroup takes (head h, partition p, chunk z): the sequences of a
// group of group_size consecutive ones, or, when group_size exceeds the G
// states the registers hold, one of its ceil(group_size / G) near-equal
// chunks: sequences s0 .. s0 + gn - 1.  A logical block that
// every sequence of the chunk maps to the same physical block, before any
// sequence's last block, is loaded once and reduced into every sequence's
// state; every other block is loaded for its sequence alone.  Each
// sequence's arithmetic is exactly that of paged_decode_kernel: wave w takes
// the same blocks w, w + NW, ... in the same order, each lane the same rows
// and columns, with the same online-softmax steps and the same merges, so
// its output and partials are bitwise the per-sequence kernel's.  The q
// slices (pre-scaled) wait in LDS; of the G states, max and sum stay in
// registers and the weighted V of each lane and sequence sits in LDS (64 KiB
// per workgroup at 16-bit), loaded around each reduction into it.  That holds
// the kernel to 128 VGPRs, so two workgroups share a CU.
// APPEND: the step's new tokens are written by this kernel, as in the
// per-sequence kernel's appending instance (see below).
// Pools hold the q format (F32 / F16 / BF16).
template <int QFMT, int CFMT, int D, int BS, int NW, int PART_BLOCKS, int G, bool APPEND>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void paged_decode_group_kernel(
    void* __restrict__ out, const void* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int S, int H, int MB, int NB, int group_size, float q_mult,
    float out_mult, float* __restrict__ ws_ml, float* __restrict__ ws_acc, int max_parts,
    const void* __restrict__ new_k, const void* __restrict__ new_v, const int32_t* __restrict__ slot_mapping) {
  using T = Tile<CFMT, D>;
  constexpr int EPL = T::EPL, LPR = T::LPR, RPL = T::RPL, EB = T::EB, ACT = T::ACT;
  constexpr int LPB = BS / RPL;
  constexpr int LPS = LPB < 4 ? LPB : 4;
  constexpr int SUB = LPB / LPS;
  constexpr int MAXB = PART_BLOCKS / NW;
  static_assert(!scaled_format(CFMT) && QFMT == CFMT, "the grouped decode reads pools in the q format");
  static_assert(MAXB <= 32 && G <= 16, "slot and sequence masks are 32 bits");
  // register load stages: two where they fit in the 128 VGPRs beside the
  // rest (f32, and f16 at head size 64 or 128, whose conversions fold into
  // mixed-precision FMAs; of the appending instances, whose loads choose
  // between the pool and the new rows, only f16 at block size 16), else one,
  // which needs about 30 fewer (checked: no instance spills)
  constexpr int ST = ((QFMT == F32 && !APPEND) ||
                      (QFMT == F16 && (D == 64 || D == 128) && (!APPEND || BS == 16))) ? 2 : 1;

  const int h = blockIdx.x;
  const int p = blockIdx.y;
  const int nchunks = (group_size + G - 1) / G;
  const int chunk = (group_size + nchunks - 1) / nchunks;
  const int zc = blockIdx.z % nchunks;
  const int s0 = (blockIdx.z / nchunks) * group_size + zc * chunk;
  const int gn = min(min(chunk, group_size - zc * chunk), S - s0);   // sequences here
  if (gn <= 0) return;                          // a chunk past the batch's last sequence
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = lane / LPR;
  const int col = lane % LPR;
  const bool col_ok = ACT == LPR || col < ACT;

  // the group's lengths, clamped as in the per-sequence kernel
  int n[G], nblocks[G], nparts[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    n[i] = i < gn ? min(max(context_lens[s0 + i], 0), MB * BS) : 0;
    nblocks[i] = (n[i] + BS - 1) / BS;
    nparts[i] = (nblocks[i] + PART_BLOCKS - 1) / PART_BLOCKS;
  }
  const int blk_begin = p * PART_BLOCKS;
  // Lane k < MAXB of each wave holds the block id of every sequence of the
  // chunk at the wave's slot k (logical block blk_begin + wave + NW k); the
  // block loop takes its ids from these lanes.  Entries past a sequence's
  // last block are read (they lie inside its table row) but never used.
  const int j_lane = blk_begin + wave + NW * lane;
  int32_t ids[G];
#pragma unroll
  for (int i = 0; i < G; ++i)
    ids[i] = (i < gn && lane < MAXB && j_lane < MB) ? block_tables[(size_t)(s0 + i) * MB + j_lane] : 0;

  // The pre-scaled q slices of the chunk wait in LDS (the same products the
  // per-sequence kernel keeps in registers).
  __shared__ float s_q[G][D];
  for (int x = threadIdx.x; x < G * D; x += NW * 64) {
    const int i = x / D, d = x % D;
    s_q[i][d] = i < gn ? load_elem<QFMT>(q, ((size_t)(s0 + i) * H + h) * D + d) * q_mult : 0.0f;
  }

  // APPEND: sequence i's new token (head h) goes to slot_mapping[s0 + i],
  // the slot of position n - 1, exactly as the cache write stores it; bit i
  // of wmask marks a slot inside the pool (padding and out-of-pool slots are
  // skipped, as by the cache write).  The lanes that read position n - 1 load
  // that row from new_k / new_v in place of the pool (see issue): the bytes
  // the write stores, so the arithmetic of write-then-decode.  The workgroup
  // of the partition that holds the sequence's last block (partition 0 when
  // n = 0) stores it, at once: no read of that slot depends on the store,
  // since no other sequence maps the block (copy-on-write).
  uint32_t wmask = 0u, smask = 0u;          // smask: the rows this workgroup stores
  if constexpr (APPEND) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (i < gn) {
        const int slot = slot_mapping[s0 + i];
        if (slot >= 0 && slot / BS < NB) {
          wmask |= 1u << i;
          if (p == (nparts[i] > 0 ? nparts[i] - 1 : 0)) smask |= 1u << i;
        }
      }
    }
    for (int x = threadIdx.x; x < G * ACT; x += NW * 64) {
      const int i = x / ACT, c = x % ACT;
      if (!((smask >> i) & 1u)) continue;
      const size_t src = (((size_t)(s0 + i) * H + h) * D + (size_t)c * EPL) * EB;
      const u32x4 kw = load16((const char*)new_k + src);
      const u32x4 vw = load16((const char*)new_v + src);
      {
        const int slot = slot_mapping[s0 + i];
        const size_t dst = (tile_base<D, BS>(slot / BS, h, H) + (size_t)(slot % BS) * D + (size_t)c * EPL) * EB;
        __builtin_nontemporal_store(kw, reinterpret_cast<u32x4*>((char*)const_cast<void*>(k_cache) + dst));
        __builtin_nontemporal_store(vw, reinterpret_cast<u32x4*>((char*)const_cast<void*>(v_cache) + dst));
      }
    }
  }

  // Blocks that may be shared: those before every sequence's last block (so
  // a shared block is full in every sequence).  Bit k of shmask: the wave's
  // slot k maps to one physical block in every sequence of the chunk.
  int cap = gn > 1 ? MB : 0;
#pragma unroll
  for (int i = 0; i < G; ++i)
    if (i < gn) cap = min(cap, n[i] > 0 ? (n[i] - 1) / BS : 0);
  bool same = lane < MAXB && j_lane < cap;
#pragma unroll
  for (int i = 1; i < G; ++i)
    if (i < gn) same = same && ids[i] == ids[0];
  const uint32_t shmask = (uint32_t)__builtin_amdgcn_ballot_w64(same);
  __syncthreads();

  // sequences without a token (n = 0): zeros
  if (p == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (i < gn && n[i] == 0) {
        const size_t ob = ((size_t)(s0 + i) * H + h) * D;
        for (int d = threadIdx.x; d < D; d += NW * 64) store_elem<QFMT>(out, ob + d, 0.0f);
      }
    }
  }

  // the group's sequences with a block at logical block j of this partition
  auto present = [&](int j) -> uint32_t {
    uint32_t b = 0u;
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (i < gn && j < min(blk_begin + PART_BLOCKS, nblocks[i])) b |= 1u << i;
    return b;
  };
  // the value of sequence c (selected without indexing registers)
  auto pick = [&](const int (&a)[G], int c) -> int {
    int r = 0;
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (i == c) r = a[i];
    return r;
  };

  const char* kbase = (const char*)k_cache;
  const char* vbase = (const char*)v_cache;
  const size_t lane_off = ((size_t)rg * D + (size_t)col * EPL) * EB;

  float m[G], l[G];
  // Each lane's weighted-V state of sequence i: EPL floats of LDS of its own
  // (no other lane touches them before the merge), as EPL / 4 16-byte chunks
  // that lie 1 KiB apart, chunk c of the wave's 64 lanes side by side, so
  // that a wave's chunk reads and writes are conflict-free.  After the block
  // loop the lanes of row group 0 store the wave's merged state the same way.
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  static_assert(EPL % 4 == 0, "states go in 16-byte chunks");
  __shared__ __attribute__((aligned(16))) f32x4 s_st[NW][G][EPL / 4][64];
  auto acc_load = [&](int i, float (&a)[EPL]) {
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c) {
      const f32x4 v = s_st[wave][i][c][lane];
#pragma unroll
      for (int k = 0; k < 4; ++k) a[4 * c + k] = v[k];
    }
  };
  auto acc_store = [&](int i, const float (&a)[EPL]) {
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c) s_st[wave][i][c][lane] = f32x4{a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
  };
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
    float z0[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) z0[e] = 0.0f;
    acc_store(i, z0);
  }

  // A unit is one sub-tile of one block, for one sequence (c >= 0) or for
  // the whole group (c = -1, a shared block).  Units go slot by slot
  // (ascending logical block), within a slot sequence by sequence, so each
  // sequence meets its blocks in the per-sequence kernel's order.  ST
  // register stages: with two, a unit's loads are issued before the previous
  // unit is reduced, as in the per-sequence kernel.
  u32x4 kc[ST][LPS], vc[ST][LPS];
  auto issue = [&](auto stc, int k, int c, int sub) {
    constexpr int st = decltype(stc)::value;
    const int j = blk_begin + wave + NW * k;
    int64_t phys = __builtin_amdgcn_readlane(pick(ids, c < 0 ? 0 : c), k);
    if ((uint64_t)phys >= (uint64_t)NB) phys = 0;    // out-of-range id: stay inside the pool
    const size_t tb = tile_base<D, BS>(phys, h, H) * EB + lane_off + (size_t)sub * LPS * RPL * D * EB;
    // APPEND, the last block of a sequence whose new token is written: the
    // lanes of row n - 1 read that row from new_k / new_v instead
    int new_row = -1;                          // local row index 0 .. LPS - 1, or -1
    size_t new_src = 0;
    if constexpr (APPEND) {
      if (c >= 0 && ((wmask >> c) & 1u) && j == pick(nblocks, c) - 1) {   // wave-uniform
        const int r = pick(n, c) - 1 - (j * BS + sub * LPS * RPL + rg);
        if (r >= 0 && r % RPL == 0 && r / RPL < LPS) {
          new_row = r / RPL;
          new_src = (((size_t)(s0 + c) * H + h) * D + (size_t)col * EPL) * EB;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const char* src = (APPEND && i == new_row) ? (const char*)new_k + new_src : kbase + tb + (size_t)i * RPL * D * EB;
      kc[st][i] = col_ok ? load16(src) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const char* src = (APPEND && i == new_row) ? (const char*)new_v + new_src : vbase + tb + (size_t)i * RPL * D * EB;
      vc[st][i] = col_ok ? load16(src) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // the per-sequence kernel's reduction of one unit into sequence i's state
  auto reduce_into = [&](auto stc, int i, int j, int sub, bool last) {
    constexpr int st = decltype(stc)::value;
    float qv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = col_ok ? s_q[i][col * EPL + e] : 0.0f;
    float z[LPS];
#pragma unroll
    for (int r = 0; r < LPS; ++r) {
      float kf[EPL];
      Chunk<CFMT>::to_f32(kc[st][r], kf);
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[e], kf[e], dot);
      z[r] = group_sum<LPR>(dot);
    }
    if (last) {                                // wave-uniform: the sequence's last block
      const int t0 = j * BS + sub * LPS * RPL + rg;
#pragma unroll
      for (int r = 0; r < LPS; ++r) {
        if (t0 + r * RPL >= n[i]) {
          z[r] = -INFINITY;
          vc[st][r] = u32x4{0u, 0u, 0u, 0u};   // rows past n may hold anything
        }
      }
    }
    float zmax = z[0];
#pragma unroll
    for (int r = 1; r < LPS; ++r) zmax = fmaxf(zmax, z[r]);
    const float m_new = fmaxf(m[i], zmax);
    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m[i] - m_ref);
    float acc[EPL];
    acc_load(i, acc);
    l[i] *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int r = 0; r < LPS; ++r) {
      const float pr = __builtin_amdgcn_exp2f(z[r] - m_ref);
      l[i] += pr;
      float vf[EPL];
      Chunk<CFMT>::to_f32(vc[st][r], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(pr, vf[e], acc[e]);
    }
    acc_store(i, acc);
    m[i] = m_new;
  };
  // A shared block (full in every sequence, never an appending one) into the
  // state of sequences i0 .. i0 + GH - 1.  Per sequence the operations and
  // their order are those of reduce_into.  All the sequences' scores come
  // first, so each K row is converted once per pass; then, sequence by
  // sequence, the rescale and the rows of V, around one load and one store
  // of that sequence's weighted V.
  constexpr int GH = G < 4 ? G : 4;            // sequences per pass of a shared block
  auto reduce_shared_part = [&](auto stc, auto basec) {
    constexpr int st = decltype(stc)::value;
    constexpr int i0 = decltype(basec)::value;
    float z[G][LPS];
#pragma unroll
    for (int i = i0; i < i0 + GH; ++i) {
      float qv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[e] = col_ok ? s_q[i][col * EPL + e] : 0.0f;
#pragma unroll
      for (int r = 0; r < LPS; ++r) {
        float kf[EPL];
        Chunk<CFMT>::to_f32(kc[st][r], kf);
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[e], kf[e], dot);
        z[i][r] = group_sum<LPR>(dot);
      }
    }
#pragma unroll
    for (int i = i0; i < i0 + GH; ++i) {
      float zmax = z[i][0];
#pragma unroll
      for (int r = 1; r < LPS; ++r) zmax = fmaxf(zmax, z[i][r]);
      const float m_new = fmaxf(m[i], zmax);
      const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_ref);
      float acc[EPL];
      acc_load(i, acc);
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
      m[i] = m_new;
#pragma unroll
      for (int r = 0; r < LPS; ++r) {
        float vf[EPL];
        Chunk<CFMT>::to_f32(vc[st][r], vf);
        const float pr = __builtin_amdgcn_exp2f(z[i][r] - m_ref);
        l[i] += pr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(pr, vf[e], acc[e]);
      }
      acc_store(i, acc);
    }
  };
  auto consume = [&](auto stc, int k, int c, int sub) {
    constexpr int st = decltype(stc)::value;
    const int j = blk_begin + wave + NW * k;
    if (c < 0) {
      reduce_shared_part(stc, std::integral_constant<int, 0>{});
      if constexpr (G > GH) {
        if (gn > GH) reduce_shared_part(stc, std::integral_constant<int, GH>{});
      }
      static_assert(G <= 2 * GH, "a shared block takes at most two passes");
      return;
    }
    const bool last = j >= min(blk_begin + PART_BLOCKS, pick(n, c) / BS);
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (i == c) reduce_into(stc, i, j, sub, last);
  };

  // the first unit at slot k or later (false at the end)
  auto seek = [&](int& k, int& c) -> bool {
    for (; k < MAXB; ++k) {
      if ((shmask >> k) & 1u) { c = -1; return true; }
      const uint32_t pm = present(blk_begin + wave + NW * k);
      if (pm) { c = __builtin_ctz(pm); return true; }
    }
    return false;
  };
  // the unit after (k, c, sub)
  auto advance = [&](int& k, int& c, int& sub) -> bool {
    if (++sub < SUB) return true;
    sub = 0;
    if (c >= 0) {
      const uint32_t pm = present(blk_begin + wave + NW * k) & ~((2u << c) - 1u);
      if (pm) { c = __builtin_ctz(pm); return true; }
    }
    ++k;
    return seek(k, c);
  };

  using S0 = std::integral_constant<int, 0>;
  int ka = 0, ca = 0, sa = 0;
  bool more = seek(ka, ca);
  if constexpr (ST == 1) {
    while (more) {
      issue(S0{}, ka, ca, sa);
      consume(S0{}, ka, ca, sa);
      more = advance(ka, ca, sa);
    }
  } else {
    using S1 = std::integral_constant<int, ST - 1>;
    if (more) issue(S0{}, ka, ca, sa);
    while (more) {
      int kb = ka, cb = ca, sb = sa;
      const bool more_b = advance(kb, cb, sb);
      if (more_b) issue(S1{}, kb, cb, sb);
      consume(S0{}, ka, ca, sa);
      if (!more_b) break;
      ka = kb; ca = cb; sa = sb;
      more = advance(ka, ca, sa);
      if (more) issue(S0{}, ka, ca, sa);
      consume(S1{}, kb, cb, sb);
    }
  }

  // every sequence's merges, as in the per-sequence kernel: row groups by
  // shuffles, then the waves through LDS, all sequences of the chunk in one
  // pass (one barrier, one output element per thread)
  __shared__ float s_m[G][NW], s_l[G][NW];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (i >= gn || p >= nparts[i]) continue;   // uniform over the workgroup
    float acc[EPL];
    acc_load(i, acc);
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      const float m_o = __shfl_xor(m[i], off);
      const float l_o = __shfl_xor(l[i], off);
      const float m_new = fmaxf(m[i], m_o);
      const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
      const float a = __builtin_amdgcn_exp2f(m[i] - m_ref), b = __builtin_amdgcn_exp2f(m_o - m_ref);
      l[i] = __builtin_fmaf(l[i], a, l_o * b);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float acc_o = __shfl_xor(acc[e], off);
        acc[e] = __builtin_fmaf(acc[e], a, acc_o * b);
      }
      m[i] = m_new;
    }
    if (lane < ACT) acc_store(i, acc);        // column d = lane * EPL + e
    if (lane == 0) { s_m[i][wave] = m[i]; s_l[i][wave] = l[i]; }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < G * D; x += NW * 64) {
    const int i = x / D, d = x % D;
    const int np = pick(nparts, i);
    if (i >= gn || p >= np) continue;
    float M = s_m[i][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[i][w]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[i][w] - M);
      L = __builtin_fmaf(s_l[i][w], f, L);
      A = __builtin_fmaf(s_st[w][i][(d % EPL) / 4][d / EPL][d % 4], f, A);
    }
    const int sq = s0 + i;
    if (np == 1) {
      store_elem<QFMT>(out, ((size_t)sq * H + h) * D + d, (A / L) * out_mult);
    } else {
      const size_t part = ((size_t)sq * H + h) * max_parts + p;
      ws_acc[part * D + d] = A;
      if (d == 0) { ws_ml[2 * part] = M; ws_ml[2 * part + 1] = L; }
    }
  }
}

// Merge the partitions of each (sequence, head) in one pass over them:
// out = sum_p A_p 2^(M_p - M) / sum_p L_p 2^(M_p - M), M the largest M_p,
// times the V scale for 8-bit pools (the pool's, or the head's from
// v_scales).  Partition p < nparts always holds at least one token, so every
// M_p is finite.
template <int QFMT, int D, int BS, int PART_TOKENS>
__global__ __launch_bounds__(D) void paged_decode_reduce_kernel(
    void* __restrict__ out, const int32_t* __restrict__ context_lens, int H, int MB, float out_mult,
    const float* __restrict__ v_scales, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    int max_parts) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  if (v_scales) out_mult *= v_scales[h];
  const int n = min(max(context_lens[s], 0), MB * BS);
  const int nparts = (n + PART_TOKENS - 1) / PART_TOKENS;
  if (nparts <= 1) return;                     // written by the partition kernel
  const size_t sh = (size_t)s * H + h;
  const float* ml = ws_ml + 2 * sh * max_parts;
  const float* acc = ws_acc + sh * max_parts * D;
  float M = ml[0], L = ml[1], A = acc[d];
  for (int p = 1; p < nparts; ++p) {
    const float mp = ml[2 * p], lp = ml[2 * p + 1], ap = acc[(size_t)p * D + d];
    const float Mn = fmaxf(M, mp);
    const float a = __builtin_amdgcn_exp2f(M - Mn), b = __builtin_amdgcn_exp2f(mp - Mn);
    L = __builtin_fmaf(L, a, lp * b);
    A = __builtin_fmaf(A, a, ap * b);
    M = Mn;
  }
  store_elem<QFMT>(out, sh * D + d, (A / L) * out_mult);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

// Waves per workgroup (8 measured best against 4 and 16).
constexpr int kWaves = 8;

// Sequence states one grouped workgroup holds.  Four, and a larger group
// runs as near-equal chunks of at most four (each chunk reads the blocks its
// sequences share once; the chunks of one group and head run on one XCD at
// the same time, so its L2 serves most repeats).  With eight states in
// registers the kernel needed 256 VGPRs and spilled; with four, and their
// weighted V in LDS, two workgroups share a CU.
constexpr int kGroupStates = 4;

template <int QFMT, int CFMT, int D, int BS>
struct DecodeLaunch {
  static constexpr int PB = part_blocks(BS);
  static_assert(PB * BS == kPartTokens, "partition must be whole blocks");
  static int max_parts(const DecodeArgs& a) { return (a.MB + PB - 1) / PB; }
  static hipError_t partitions(const DecodeArgs& a, hipStream_t st) {
    const int P = max_parts(a);
    if constexpr (!scaled_format(CFMT)) {
      if (a.group_size > 1) {
        // one workgroup per (head, partition, group of sequences or chunk of one)
        constexpr int G = kGroupStates;
        dim3 ggrid(a.H, P, (a.S + a.group_size - 1) / a.group_size * ((a.group_size + G - 1) / G));
        if (a.slot_mapping) {
          hipLaunchKernelGGL((paged_decode_group_kernel<QFMT, CFMT, D, BS, kWaves, PB, G, true>), ggrid,
                             dim3(kWaves * 64), 0, st, a.out, a.q, a.k_cache, a.v_cache, a.block_tables,
                             a.context_lens, a.S, a.H, a.MB, a.NB, a.group_size, a.q_mult, a.out_mult, a.ws_ml,
                             a.ws_acc, P, a.new_k, a.new_v, a.slot_mapping);
        } else {
          hipLaunchKernelGGL((paged_decode_group_kernel<QFMT, CFMT, D, BS, kWaves, PB, G, false>), ggrid,
                             dim3(kWaves * 64), 0, st, a.out, a.q, a.k_cache, a.v_cache, a.block_tables,
                             a.context_lens, a.S, a.H, a.MB, a.NB, a.group_size, a.q_mult, a.out_mult, a.ws_ml,
                             a.ws_acc, P, nullptr, nullptr, nullptr);
        }
        return hipGetLastError();
      }
    }
    // head-major: the workgroups that run together read the H tiles of the
    // same physical blocks, one contiguous [H][BS][D] span
    dim3 grid(a.H, P, a.S);
    if (a.slot_mapping) {
      if constexpr (scaled_format(CFMT)) {
        // 8-bit pools: the write's quantisation (an IEEE division and an
        // encoding per element) would cost the partition kernel registers
        // and occupancy, so the cache-write kernel runs first instead
        const hipError_t e = launch_reshape_and_cache(a.new_k, a.new_v, const_cast<void*>(a.k_cache),
                                                      const_cast<void*>(a.v_cache), a.slot_mapping, a.S, a.H,
                                                      D, BS, a.NB, QFMT, CFMT, a.k_scale, a.v_scale, a.k_scales,
                                                      a.v_scales, st);
        if (e != hipSuccess) return e;
      } else {
        hipLaunchKernelGGL((paged_decode_kernel<QFMT, CFMT, D, BS, kWaves, PB, true>), grid, dim3(kWaves * 64), 0,
                           st, a.out, a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.H, a.MB, a.NB,
                           a.q_mult, a.out_mult, a.k_scales, a.v_scales, a.ws_ml, a.ws_acc, P, a.new_k, a.new_v,
                           a.slot_mapping);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((paged_decode_kernel<QFMT, CFMT, D, BS, kWaves, PB, false>), grid, dim3(kWaves * 64), 0, st,
                       a.out, a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.H, a.MB, a.NB, a.q_mult,
                       a.out_mult, a.k_scales, a.v_scales, a.ws_ml, a.ws_acc, P, nullptr, nullptr, nullptr);
    return hipGetLastError();
  }
  static hipError_t merge(const DecodeArgs& a, hipStream_t st) {
    const int P = max_parts(a);
    if (P == 1) return hipSuccess;             // every sequence fits one partition
    hipLaunchKernelGGL((paged_decode_reduce_kernel<QFMT, D, BS, PB * BS>), dim3(a.H, a.S), dim3(D), 0, st,
                       a.out, a.context_lens, a.H, a.MB, a.out_mult, a.v_scales, a.ws_ml, a.ws_acc, P);
    return hipGetLastError();
  }
};

// dispatch on (q, cache) formats, head size and block size
template <template <int, int, int, int> class L, int Q, int C, int D>
static hipError_t dispatch_bs(const DecodeArgs& a, bool merge, hipStream_t st) {
  if (a.BS == 16) return merge ? L<Q, C, D, 16>::merge(a, st) : L<Q, C, D, 16>::partitions(a, st);
  return merge ? L<Q, C, D, 32>::merge(a, st) : L<Q, C, D, 32>::partitions(a, st);
}

template <template <int, int, int, int> class L, int Q, int C>
static hipError_t dispatch_shape(const DecodeArgs& a, bool merge, hipStream_t st) {
  switch (a.D) {
    case 64: return dispatch_bs<L, Q, C, 64>(a, merge, st);
    case 80: return dispatch_bs<L, Q, C, 80>(a, merge, st);
    case 96: return dispatch_bs<L, Q, C, 96>(a, merge, st);
    case 128: return dispatch_bs<L, Q, C, 128>(a, merge, st);
    case 256: return dispatch_bs<L, Q, C, 256>(a, merge, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t dispatch_decode(const DecodeArgs& a, bool merge, hipStream_t st) {
  if (a.q_fmt == F32 && a.c_fmt == F32) return dispatch_shape<DecodeLaunch, F32, F32>(a, merge, st);
  if (a.q_fmt == F16 && a.c_fmt == F16) return dispatch_shape<DecodeLaunch, F16, F16>(a, merge, st);
  if (a.q_fmt == BF16 && a.c_fmt == BF16) return dispatch_shape<DecodeLaunch, BF16, BF16>(a, merge, st);
  if (a.q_fmt == F16 && a.c_fmt == E4M3) return dispatch_shape<DecodeLaunch, F16, E4M3>(a, merge, st);
  if (a.q_fmt == BF16 && a.c_fmt == E4M3) return dispatch_shape<DecodeLaunch, BF16, E4M3>(a, merge, st);
  if (a.q_fmt == F16 && a.c_fmt == I8) return dispatch_shape<DecodeLaunch, F16, I8>(a, merge, st);
  if (a.q_fmt == BF16 && a.c_fmt == I8) return dispatch_shape<DecodeLaunch, BF16, I8>(a, merge, st);
  return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_partitions(const DecodeArgs& a, hipStream_t st) {
  return dispatch_decode(a, false, st);
}

hipError_t launch_paged_decode_merge(const DecodeArgs& a, hipStream_t st) {
  return dispatch_decode(a, true, st);
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t st) {
  const hipError_t e = dispatch_decode(a, false, st);
  return e != hipSuccess ? e : dispatch_decode(a, true, st);
}

}  // namespace pkv

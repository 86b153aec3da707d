// Device helpers shared by the gfx950 kernels of libpagedkv: element formats,
// 16-byte vector loads, wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Element formats (values match pkv_dtype in include/pagedkv.h).
enum Fmt : int { F32 = 0, F16 = 1, BF16 = 2, E4M3 = 3, I8 = 4 };

template <int FMT> struct FmtInfo;
template <> struct FmtInfo<F32>  { static constexpr int bytes = 4; };
template <> struct FmtInfo<F16>  { static constexpr int bytes = 2; };
template <> struct FmtInfo<BF16> { static constexpr int bytes = 2; };
template <> struct FmtInfo<E4M3> { static constexpr int bytes = 1; };
template <> struct FmtInfo<I8>   { static constexpr int bytes = 1; };

// formats that store x / scale with one fp32 scale per pool
constexpr bool scaled_format(int fmt) { return fmt == E4M3 || fmt == I8; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).x;
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).y;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rn(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_rn(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Two E4M3FN bytes (bytes 2*sel, 2*sel+1 of w) -> two floats, with gfx950's
// fp8 conversion instruction (OCP E4M3FN on this target).
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// ---------------------------------------------------------------------------
// 16-byte chunk -> floats
// ---------------------------------------------------------------------------

template <int FMT> struct Chunk;

template <> struct Chunk<F32> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void to_f32(const u32x4& c, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(c[i]);
  }
};
template <> struct Chunk<F16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void to_f32(const u32x4& c, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = f16_lo(c[i]); o[2 * i + 1] = f16_hi(c[i]); }
  }
};
template <> struct Chunk<BF16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void to_f32(const u32x4& c, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(c[i]); o[2 * i + 1] = bf16_hi(c[i]); }
  }
};
template <> struct Chunk<E4M3> {
  static constexpr int n = 16;
  __device__ __forceinline__ static void to_f32(const u32x4& c, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 a = e4m3x2_to_f32<false>(c[i]);
      const f32x2 b = e4m3x2_to_f32<true>(c[i]);
      o[4 * i + 0] = a.x; o[4 * i + 1] = a.y; o[4 * i + 2] = b.x; o[4 * i + 3] = b.y;
    }
  }
};

// INT8 bytes come out offset: each byte b is read as the unsigned value
// u = b + 128 (its sign bit flipped), one v_cvt_f32_ubyte per element.  The
// user subtracts 128 where it is cheap: once per dot product
// (sum q*b = sum q*u - 128 sum q) and once per softmax-weighted sum
// (sum p*b = sum p*u - 128 sum p).
template <> struct Chunk<I8> {
  static constexpr int n = 16;
  static constexpr float offset = 128.0f;
  __device__ __forceinline__ static void to_f32(const u32x4& c, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = c[i] ^ 0x80808080u;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[4 * i + k] = (float)((w >> (8 * k)) & 0xFFu);
    }
  }
};

// q / out element access for the three query formats
template <int FMT> __device__ __forceinline__ float load_elem(const void* p, size_t i);
template <> __device__ __forceinline__ float load_elem<F32>(const void* p, size_t i) {
  return ((const float*)p)[i];
}
template <> __device__ __forceinline__ float load_elem<F16>(const void* p, size_t i) {
  return (float)((const _Float16*)p)[i];
}
template <> __device__ __forceinline__ float load_elem<BF16>(const void* p, size_t i) {
  return __uint_as_float(((uint32_t)((const uint16_t*)p)[i]) << 16);
}

template <int FMT> __device__ __forceinline__ void store_elem(void* p, size_t i, float v);
template <> __device__ __forceinline__ void store_elem<F32>(void* p, size_t i, float v) {
  ((float*)p)[i] = v;
}
template <> __device__ __forceinline__ void store_elem<F16>(void* p, size_t i, float v) {
  ((uint16_t*)p)[i] = f32_to_f16_rn(v);
}
template <> __device__ __forceinline__ void store_elem<BF16>(void* p, size_t i, float v) {
  ((uint16_t*)p)[i] = f32_to_bf16_rn(v);
}

// Element offset of the (block, head) tile in a [NB][H][BS][D] pool: the one
// address rule every kernel that touches a pool uses.
template <int D, int BS>
__device__ __forceinline__ size_t tile_base(int64_t block, int h, int H) {
  return ((size_t)block * (size_t)H + (size_t)h) * (size_t)(BS * D);
}

// 16-byte global load, marked non-temporal: the K/V stream is read once,
// with no reuse expected in the caches.
__device__ __forceinline__ u32x4 load16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// wave64 cross-lane reductions
// ---------------------------------------------------------------------------

// DPP controls (GCN/CDNA encoding)
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G in {1,2,4,8,16,32,64}); every lane
// of a group receives the group's sum.  After the quad steps every lane of a
// quad holds the quad sum, so the mirrors pair quads (8) and half-rows (16).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (G >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (G >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (G >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  if constexpr (G >= 64) x += __shfl_xor(x, 32);
  return x;
}

}  // namespace pkv

// C ABI of libpagedkv (declared in include/pagedkv.h): host-side argument
// checks, dtype/shape dispatch and workspace layout.  Nothing here allocates
// or keeps state (pkv_paged_attention_decode_static takes the static buffer
// of decode_static.hip); only pkv_check_step_inputs synchronises (it reads
// its result back).

#include <cmath>
#include <cstdint>

#include "pagedkv.h"
#include "checks.h"
#include "decode_static.h"
#include "kernels.h"

namespace {

constexpr int kVersion = 800;  // 0.8.0

bool ok_head_size(int32_t D) { return D == 64 || D == 80 || D == 96 || D == 128 || D == 256; }
bool ok_block_size(int32_t BS) { return BS == 16 || BS == 32; }
// the prompt kernel's head sizes (its launcher dispatches exactly these)
bool ok_prefill_head_size(int32_t D) { return D == 64 || D == 80 || D == 96 || D == 128 || D == 256; }
bool ok_dtype(int v) { return v >= PKV_F32 && v <= PKV_INT8; }
bool scaled(int fmt) { return fmt == PKV_FP8_E4M3 || fmt == PKV_INT8; }

// (query / source dtype, cache dtype) pairs with a kernel
bool ok_pair(int q, int c) {
  return (q == PKV_F32 && c == PKV_F32) || (q == PKV_F16 && c == PKV_F16) ||
         (q == PKV_BF16 && c == PKV_BF16) || ((q == PKV_F16 || q == PKV_BF16) && scaled(c));
}

bool ok_scale(float x) { return std::isfinite(x) && x > 0.0f; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int fmt) { return fmt == PKV_F32 ? 4 : scaled(fmt) ? 1 : 2; }

constexpr int32_t kMaxGridYZ = 65535;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Partitions per sequence the decode's grid provides for tables of MB blocks
// of BS tokens (MB, BS > 0).
int32_t decode_max_parts(int32_t MB, int32_t BS) {
  const int64_t pb = BS < pkv::kPartTokens ? pkv::kPartTokens / BS : 1;
  return (int32_t)(((int64_t)MB + pb - 1) / pb);     // in 64 bits: MB may be near INT32_MAX
}

pkv_status from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// The address a kernel may use for p, or nullptr: device memory as it is,
// pinned host memory through its device mapping; pageable host memory (or an
// address HIP does not know) has none.
void* kernel_address(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();                 // clear the error the query leaves behind
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) return const_cast<void*>(p);
  if (a.type == hipMemoryTypeHost) return a.devicePointer;
  return nullptr;
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_DEVICE_CHECK: return "device-side input check failed";
    default: break;
  }
  return "unknown status";
}

int pkv_version(void) { return kVersion; }

}  // extern "C"

namespace {

// The per-head scale arrays of an 8-bit pool: both given, 4-byte aligned.
// Other pools ignore them.
pkv_status check_head_scales(int cache_dtype, const float* k_scales, const float* v_scales) {
  if (!scaled(cache_dtype)) return PKV_OK;
  if (!k_scales || !v_scales || !aligned(k_scales, 4) || !aligned(v_scales, 4)) return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

pkv_status reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int32_t T, int32_t H, int32_t D, int32_t BS, int32_t NB,
                             pkv_dtype src_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
                             const float* k_scales, const float* v_scales, bool head, hipStream_t stream) {
  if (T < 0 || H <= 0 || D <= 0 || BS <= 0 || NB <= 0) return PKV_ERR_INVALID_ARG;
  if (!ok_dtype(src_dtype) || !ok_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!ok_scale(k_scale) || !ok_scale(v_scale)) return PKV_ERR_INVALID_ARG;
  if (!ok_head_size(D) || !ok_block_size(BS) || !ok_pair(src_dtype, cache_dtype))
    return PKV_ERR_UNSUPPORTED;
  if (T == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PKV_ERR_INVALID_ARG;
  if (head) {
    const pkv_status st = check_head_scales(cache_dtype, k_scales, v_scales);
    if (st != PKV_OK) return st;
  }
  const bool per_head = head && scaled(cache_dtype);
  return from_hip(pkv::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, T, H, D,
                                                BS, NB, src_dtype, cache_dtype, k_scale, v_scale,
                                                per_head ? k_scales : nullptr, per_head ? v_scales : nullptr,
                                                stream));
}

}  // namespace

extern "C" {

pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int32_t T, int32_t H, int32_t D,
                                 int32_t BS, int32_t NB, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                 float k_scale, float v_scale, hipStream_t stream) {
  return reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, T, H, D, BS, NB, src_dtype, cache_dtype,
                           k_scale, v_scale, nullptr, nullptr, false, stream);
}

pkv_status pkv_reshape_and_cache_head_scales(const void* key, const void* value, void* k_cache, void* v_cache,
                                             const int32_t* slot_mapping, int32_t T, int32_t H, int32_t D,
                                             int32_t BS, int32_t NB, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                             const float* k_scales, const float* v_scales, hipStream_t stream) {
  return reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, T, H, D, BS, NB, src_dtype, cache_dtype,
                           1.0f, 1.0f, k_scales, v_scales, true, stream);
}

size_t pkv_decode_workspace_bytes(int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB) {
  if (S <= 0 || H <= 0 || D <= 0 || BS <= 0 || MB <= 0) return 0;
  const size_t P = (size_t)decode_max_parts(MB, BS);
  if (P <= 1) return 0;
  const size_t parts = (size_t)S * (size_t)H * P;
  return round_up(parts * 2 * sizeof(float), 256) + parts * (size_t)D * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points; fills `a` on success.
// head: the call takes per-head scale arrays (k_scales / v_scales, fp32 [H] on
// the device) in place of k_scale / v_scale; merge_only: only v_scales is
// read.
pkv_status check_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
                        int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
                        pkv_dtype cache_dtype, float k_scale, float v_scale, const void* workspace,
                        size_t workspace_bytes, bool merge_only, pkv::DecodeArgs* a, bool head = false,
                        const float* k_scales = nullptr, const float* v_scales = nullptr) {
  if (S < 0 || H <= 0 || D <= 0 || BS <= 0 || MB <= 0 || NB <= 0) return PKV_ERR_INVALID_ARG;
  if (!ok_dtype(q_dtype) || !ok_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!ok_scale(scale) || !ok_scale(k_scale) || !ok_scale(v_scale)) return PKV_ERR_INVALID_ARG;
  if (!ok_head_size(D) || !ok_block_size(BS) || !ok_pair(q_dtype, cache_dtype))
    return PKV_ERR_UNSUPPORTED;
  // grid (H, partitions, S): each of y and z at most 65535
  if (S > kMaxGridYZ || H > kMaxGridYZ || decode_max_parts(MB, BS) > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  if (S == 0) return PKV_OK;
  if (!out || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!merge_only) {
    if (!q || !k_cache || !v_cache || !block_tables) return PKV_ERR_INVALID_ARG;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return PKV_ERR_INVALID_ARG;
  }
  if (head) {
    const pkv_status st = check_head_scales(cache_dtype, merge_only ? v_scales : k_scales, v_scales);
    if (st != PKV_OK) return st;
  }
  const size_t need = pkv_decode_workspace_bytes(S, H, D, BS, MB);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PKV_ERR_INVALID_ARG;
  }
  const size_t parts = (size_t)S * (size_t)H * (size_t)decode_max_parts(MB, BS);
  const bool fp8 = scaled(cache_dtype);
  const bool per_head = head && fp8;     // the kernels multiply in each head's scales
  a->out = out;
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->S = S;
  a->H = H;
  a->D = D;
  a->BS = BS;
  a->MB = MB;
  a->NB = NB;
  a->q_fmt = q_dtype;
  a->c_fmt = cache_dtype;
  // per-pool: (scale * log2(e)) * k_scale; per head the kernels form the same
  // product with the head's scale, so equal per-head scales give the same bits
  a->q_mult = scale * 1.4426950408889634f * (fp8 && !per_head ? k_scale : 1.0f);
  a->out_mult = fp8 && !per_head ? v_scale : 1.0f;
  a->k_scales = per_head && !merge_only ? k_scales : nullptr;
  a->v_scales = per_head ? v_scales : nullptr;
  a->group_size = 1;
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a->ws_ml = need ? reinterpret_cast<float*>(ws) : nullptr;
  a->ws_acc = need ? reinterpret_cast<float*>(ws + round_up(parts * 2 * sizeof(float), 256)) : nullptr;
  a->new_k = nullptr;
  a->new_v = nullptr;
  a->slot_mapping = nullptr;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  return PKV_OK;
}

// The appending decode's own checks, after those of the decode.
pkv_status check_append(const void* key, const void* value, const int32_t* slot_mapping, pkv::DecodeArgs* a) {
  if (!key || !value || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16)) return PKV_ERR_INVALID_ARG;
  a->new_k = key;
  a->new_v = value;
  a->slot_mapping = slot_mapping;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t S, int32_t H, int32_t D,
                                      int32_t BS, int32_t MB, int32_t NB, float scale,
                                      pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                                      float v_scale, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS,
                                     MB, NB, scale, q_dtype, cache_dtype, k_scale, v_scale, workspace,
                                     workspace_bytes, false, &a);
  if (st != PKV_OK || S == 0) return st;
  return from_hip(pkv::launch_paged_decode(a, stream));
}

pkv_status pkv_paged_attention_decode_static(void* out, const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* block_tables,
                                             const int32_t* context_lens, int32_t S, int32_t H, int32_t D,
                                             int32_t BS, int32_t MB, int32_t NB, float scale,
                                             pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                                             float v_scale, hipStream_t stream) {
  // Checked against a stand-in address first (never dereferenced): the
  // arguments and the size limit are refused before anything touches the
  // device.  The partial pointers are then moved onto the static buffer.
  char* const stand_in = reinterpret_cast<char*>(uintptr_t{256});
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS,
                                     MB, NB, scale, q_dtype, cache_dtype, k_scale, v_scale, stand_in,
                                     PKV_STATIC_WORKSPACE_BYTES, false, &a);
  if (st != PKV_OK || S == 0) return st;
  if (a.ws_ml) {
    void* ws = nullptr;
    if (pkv::static_workspace(&ws) != hipSuccess) return PKV_ERR_HIP;
    char* base = static_cast<char*>(ws);
    a.ws_ml = reinterpret_cast<float*>(base + (reinterpret_cast<char*>(a.ws_ml) - stand_in));
    a.ws_acc = reinterpret_cast<float*>(base + (reinterpret_cast<char*>(a.ws_acc) - stand_in));
  }
  return from_hip(pkv::launch_paged_decode(a, stream));
}

pkv_status pkv_paged_attention_decode_partitions(
    void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS,
                                     MB, NB, scale, q_dtype, cache_dtype, k_scale, v_scale, workspace,
                                     workspace_bytes, false, &a);
  if (st != PKV_OK || S == 0) return st;
  return from_hip(pkv::launch_paged_decode_partitions(a, stream));
}

pkv_status pkv_paged_attention_decode_append(void* out, const void* q, const void* key, const void* value,
                                             void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                             const int32_t* block_tables, const int32_t* context_lens,
                                             int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB,
                                             int32_t NB, float scale, pkv_dtype q_dtype,
                                             pkv_dtype cache_dtype, float k_scale, float v_scale,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pkv::DecodeArgs a;
  pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB,
                               scale, q_dtype, cache_dtype, k_scale, v_scale, workspace, workspace_bytes,
                               false, &a);
  if (st != PKV_OK || S == 0) return st;
  st = check_append(key, value, slot_mapping, &a);
  if (st != PKV_OK) return st;
  return from_hip(pkv::launch_paged_decode(a, stream));
}

pkv_status pkv_paged_attention_decode_append_partitions(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S,
    int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
    pkv_dtype cache_dtype, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  pkv::DecodeArgs a;
  pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB,
                               scale, q_dtype, cache_dtype, k_scale, v_scale, workspace, workspace_bytes,
                               false, &a);
  if (st != PKV_OK || S == 0) return st;
  st = check_append(key, value, slot_mapping, &a);
  if (st != PKV_OK) return st;
  return from_hip(pkv::launch_paged_decode_partitions(a, stream));
}

pkv_status pkv_paged_attention_decode_merge(void* out, const int32_t* context_lens, int32_t S,
                                            int32_t H, int32_t D, int32_t BS, int32_t MB,
                                            pkv_dtype q_dtype, pkv_dtype cache_dtype, float v_scale,
                                            const void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, nullptr, nullptr, nullptr, nullptr, context_lens, S, H, D, BS,
                                     MB, 1, 1.0f, q_dtype, cache_dtype, 1.0f, v_scale, workspace,
                                     workspace_bytes, true, &a);
  if (st != PKV_OK || S == 0) return st;
  return from_hip(pkv::launch_paged_decode_merge(a, stream));
}

}  // extern "C"

namespace {

// The decode with groups of sequences sharing block loads.
pkv_status decode_grouped(void* out, const void* q, const void* key, const void* value, void* k_cache,
                          void* v_cache, const int32_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB,
                          int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, int32_t group_size,
                          void* workspace, size_t workspace_bytes, bool partitions_only, hipStream_t stream) {
  pkv::DecodeArgs a;
  pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, scale,
                               q_dtype, cache_dtype, 1.0f, 1.0f, workspace, workspace_bytes, false, &a);
  if (st != PKV_OK) return st;
  if (group_size < 1 || group_size > pkv::kMaxGroup) return PKV_ERR_INVALID_ARG;
  if (scaled(cache_dtype)) return PKV_ERR_UNSUPPORTED;
  const bool any_new = key || value || slot_mapping;
  if (any_new && !(key && value && slot_mapping)) return PKV_ERR_INVALID_ARG;
  if (S == 0) return PKV_OK;
  if (any_new) {
    st = check_append(key, value, slot_mapping, &a);
    if (st != PKV_OK) return st;
  }
  a.group_size = group_size;
  return from_hip(partitions_only ? pkv::launch_paged_decode_partitions(a, stream)
                                  : pkv::launch_paged_decode(a, stream));
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode_grouped(void* out, const void* q, const void* key, const void* value,
                                              void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                              const int32_t* block_tables, const int32_t* context_lens, int32_t S,
                                              int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale,
                                              pkv_dtype q_dtype, pkv_dtype cache_dtype, int32_t group_size,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_grouped(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, S, H, D, BS,
                        MB, NB, scale, q_dtype, cache_dtype, group_size, workspace, workspace_bytes, false, stream);
}

pkv_status pkv_paged_attention_decode_grouped_partitions(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
    int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    int32_t group_size, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_grouped(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, S, H, D, BS,
                        MB, NB, scale, q_dtype, cache_dtype, group_size, workspace, workspace_bytes, true, stream);
}

// The decode entry points with one scale per head (8-bit pools): the same
// checks and kernels, with k_scales / v_scales in place of k_scale / v_scale.

pkv_status pkv_paged_attention_decode_head_scales(void* out, const void* q, const void* k_cache,
                                                  const void* v_cache, const int32_t* block_tables,
                                                  const int32_t* context_lens, int32_t S, int32_t H, int32_t D,
                                                  int32_t BS, int32_t MB, int32_t NB, float scale,
                                                  pkv_dtype q_dtype, pkv_dtype cache_dtype, const float* k_scales,
                                                  const float* v_scales, void* workspace, size_t workspace_bytes,
                                                  hipStream_t stream) {
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB,
                                     scale, q_dtype, cache_dtype, 1.0f, 1.0f, workspace, workspace_bytes, false,
                                     &a, true, k_scales, v_scales);
  if (st != PKV_OK || S == 0) return st;
  return from_hip(pkv::launch_paged_decode(a, stream));
}

pkv_status pkv_paged_attention_decode_partitions_head_scales(
    void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, const float* k_scales, const float* v_scales,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB,
                                     scale, q_dtype, cache_dtype, 1.0f, 1.0f, workspace, workspace_bytes, false,
                                     &a, true, k_scales, v_scales);
  if (st != PKV_OK || S == 0) return st;
  return from_hip(pkv::launch_paged_decode_partitions(a, stream));
}

pkv_status pkv_paged_attention_decode_merge_head_scales(void* out, const int32_t* context_lens, int32_t S,
                                                        int32_t H, int32_t D, int32_t BS, int32_t MB,
                                                        pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                                        const float* v_scales, const void* workspace,
                                                        size_t workspace_bytes, hipStream_t stream) {
  pkv::DecodeArgs a;
  const pkv_status st = check_decode(out, nullptr, nullptr, nullptr, nullptr, context_lens, S, H, D, BS, MB, 1,
                                     1.0f, q_dtype, cache_dtype, 1.0f, 1.0f, workspace, workspace_bytes, true, &a,
                                     true, nullptr, v_scales);
  if (st != PKV_OK || S == 0) return st;
  return from_hip(pkv::launch_paged_decode_merge(a, stream));
}

pkv_status pkv_paged_attention_decode_append_head_scales(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
    int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    const float* k_scales, const float* v_scales, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pkv::DecodeArgs a;
  pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, scale,
                               q_dtype, cache_dtype, 1.0f, 1.0f, workspace, workspace_bytes, false, &a, true,
                               k_scales, v_scales);
  if (st != PKV_OK || S == 0) return st;
  st = check_append(key, value, slot_mapping, &a);
  if (st != PKV_OK) return st;
  return from_hip(pkv::launch_paged_decode(a, stream));
}

pkv_status pkv_paged_attention_decode_append_partitions_head_scales(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t H,
    int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    const float* k_scales, const float* v_scales, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pkv::DecodeArgs a;
  pkv_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, S, H, D, BS, MB, NB, scale,
                               q_dtype, cache_dtype, 1.0f, 1.0f, workspace, workspace_bytes, false, &a, true,
                               k_scales, v_scales);
  if (st != PKV_OK || S == 0) return st;
  st = check_append(key, value, slot_mapping, &a);
  if (st != PKV_OK) return st;
  return from_hip(pkv::launch_paged_decode_partitions(a, stream));
}

}  // extern "C"

namespace {

// The prompt attention's checks; fills `a` on success (*done: nothing to enqueue).
pkv_status check_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens,
                         int32_t S, int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS, int32_t MB,
                         int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                         float v_scale, pkv::PrefillArgs* a, bool* done, bool head = false,
                         const float* k_scales = nullptr, const float* v_scales = nullptr) {
  *done = true;
  if (S < 0 || Tq < 0 || max_q_len < 0 || H <= 0 || D <= 0 || BS <= 0 || MB <= 0 || NB <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!ok_dtype(q_dtype) || !ok_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!ok_scale(scale) || !ok_scale(k_scale) || !ok_scale(v_scale)) return PKV_ERR_INVALID_ARG;
  if (!ok_prefill_head_size(D) || !ok_block_size(BS) || (q_dtype != PKV_F16 && q_dtype != PKV_BF16) ||
      (cache_dtype != q_dtype && !scaled(cache_dtype)))
    return PKV_ERR_UNSUPPORTED;
  // H as for the decode (it also keeps the appending kernel's 32-bit row
  // offsets into key / value, 32 rows of H heads, below 2^32)
  if (S > kMaxGridYZ || H > kMaxGridYZ || max_q_len > kMaxGridYZ * 128) return PKV_ERR_UNSUPPORTED;
  if (S == 0 || Tq == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !cu_q_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PKV_ERR_INVALID_ARG;
  if (head) {
    const pkv_status st = check_head_scales(cache_dtype, k_scales, v_scales);
    if (st != PKV_OK) return st;
  }
  const bool per_head = head && scaled(cache_dtype);
  a->out = out;
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->cu_q_lens = cu_q_lens;
  a->S = S;
  a->Tq = Tq;
  a->max_q_len = max_q_len;
  a->H = H;
  a->D = D;
  a->BS = BS;
  a->MB = MB;
  a->NB = NB;
  a->fmt = q_dtype;
  a->c_fmt = cache_dtype;
  a->s_mult = scale * 1.4426950408889634f * (scaled(cache_dtype) && !per_head ? k_scale : 1.0f);
  a->out_mult = scaled(cache_dtype) && !per_head ? v_scale : 1.0f;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  a->k_scales = per_head ? k_scales : nullptr;
  a->v_scales = per_head ? v_scales : nullptr;
  a->new_k = nullptr;
  a->new_v = nullptr;
  a->slot_mapping = nullptr;
  *done = false;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* cu_q_lens, int32_t S,
                                       int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS,
                                       int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
                                       pkv_dtype cache_dtype, float k_scale, float v_scale, hipStream_t stream) {
  pkv::PrefillArgs a;
  bool done;
  const pkv_status st = check_prefill(out, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, S, Tq,
                                      max_q_len, H, D, BS, MB, NB, scale, q_dtype, cache_dtype, k_scale,
                                      v_scale, &a, &done);
  if (st != PKV_OK || done) return st;
  return from_hip(pkv::launch_paged_prefill(a, stream));
}

pkv_status pkv_paged_attention_prefill_append(void* out, const void* q, const void* key, const void* value,
                                              void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              const int32_t* cu_q_lens, int32_t S, int32_t Tq,
                                              int32_t max_q_len, int32_t H, int32_t D, int32_t BS, int32_t MB,
                                              int32_t NB, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                              float k_scale, float v_scale, hipStream_t stream) {
  pkv::PrefillArgs a;
  bool done;
  const pkv_status st = check_prefill(out, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, S, Tq,
                                      max_q_len, H, D, BS, MB, NB, scale, q_dtype, cache_dtype, k_scale,
                                      v_scale, &a, &done);
  if (st != PKV_OK || done) return st;
  if (!key || !value || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16)) return PKV_ERR_INVALID_ARG;
  a.new_k = key;
  a.new_v = value;
  a.slot_mapping = slot_mapping;
  return from_hip(pkv::launch_paged_prefill(a, stream));
}

pkv_status pkv_paged_attention_prefill_head_scales(void* out, const void* q, const void* k_cache,
                                                   const void* v_cache, const int32_t* block_tables,
                                                   const int32_t* context_lens, const int32_t* cu_q_lens, int32_t S,
                                                   int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS,
                                                   int32_t MB, int32_t NB, float scale, pkv_dtype q_dtype,
                                                   pkv_dtype cache_dtype, const float* k_scales,
                                                   const float* v_scales, hipStream_t stream) {
  pkv::PrefillArgs a;
  bool done;
  const pkv_status st = check_prefill(out, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, S, Tq,
                                      max_q_len, H, D, BS, MB, NB, scale, q_dtype, cache_dtype, 1.0f, 1.0f, &a,
                                      &done, true, k_scales, v_scales);
  if (st != PKV_OK || done) return st;
  return from_hip(pkv::launch_paged_prefill(a, stream));
}

pkv_status pkv_paged_attention_prefill_append_head_scales(
    void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens,
    int32_t S, int32_t Tq, int32_t max_q_len, int32_t H, int32_t D, int32_t BS, int32_t MB, int32_t NB, float scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, const float* k_scales, const float* v_scales, hipStream_t stream) {
  pkv::PrefillArgs a;
  bool done;
  const pkv_status st = check_prefill(out, q, k_cache, v_cache, block_tables, context_lens, cu_q_lens, S, Tq,
                                      max_q_len, H, D, BS, MB, NB, scale, q_dtype, cache_dtype, 1.0f, 1.0f, &a,
                                      &done, true, k_scales, v_scales);
  if (st != PKV_OK || done) return st;
  if (!key || !value || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16)) return PKV_ERR_INVALID_ARG;
  a.new_k = key;
  a.new_v = value;
  a.slot_mapping = slot_mapping;
  return from_hip(pkv::launch_paged_prefill(a, stream));
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t N,
                           int32_t H, int32_t D, int32_t BS, int32_t NB, pkv_dtype cache_dtype,
                           hipStream_t stream) {
  if (N < 0 || H <= 0 || D <= 0 || BS <= 0 || NB <= 0) return PKV_ERR_INVALID_ARG;
  if (!ok_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!ok_head_size(D) || !ok_block_size(BS)) return PKV_ERR_UNSUPPORTED;
  if (N > (1 << 30)) return PKV_ERR_UNSUPPORTED;
  if (N == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return PKV_ERR_INVALID_ARG;
  const size_t block_bytes = (size_t)H * BS * D * elem_bytes(cache_dtype);
  return from_hip(pkv::launch_copy_blocks(k_cache, v_cache, pairs, N, NB, block_bytes, stream));
}

pkv_status pkv_swap_blocks(void* dst_k_cache, void* dst_v_cache, const void* src_k_cache,
                           const void* src_v_cache, const int32_t* pairs, int32_t N, int32_t H, int32_t D,
                           int32_t BS, int32_t NB_src, int32_t NB_dst, pkv_dtype cache_dtype,
                           hipStream_t stream) {
  if (N < 0 || H <= 0 || D <= 0 || BS <= 0 || NB_src <= 0 || NB_dst <= 0) return PKV_ERR_INVALID_ARG;
  if (!ok_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!ok_head_size(D) || !ok_block_size(BS)) return PKV_ERR_UNSUPPORTED;
  if (N > (1 << 30)) return PKV_ERR_UNSUPPORTED;
  if (N == 0) return PKV_OK;
  if (!dst_k_cache || !dst_v_cache || !src_k_cache || !src_v_cache || !pairs) return PKV_ERR_INVALID_ARG;
  void* dk = kernel_address(dst_k_cache);
  void* dv = kernel_address(dst_v_cache);
  void* sk = kernel_address(src_k_cache);
  void* sv = kernel_address(src_v_cache);
  void* pr = kernel_address(pairs);
  if (!dk || !dv || !sk || !sv || !pr) return PKV_ERR_INVALID_ARG;
  if (!aligned(dk, 16) || !aligned(dv, 16) || !aligned(sk, 16) || !aligned(sv, 16)) return PKV_ERR_INVALID_ARG;
  const size_t block_bytes = (size_t)H * BS * D * elem_bytes(cache_dtype);
  return from_hip(pkv::launch_swap_blocks(dk, dv, sk, sv, static_cast<const int32_t*>(pr), N, NB_src, NB_dst,
                                          block_bytes, stream));
}

pkv_status pkv_gather_kv(void* k_out, void* v_out, const int32_t* cu_lens, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t S, int32_t H, int32_t D, int32_t BS,
                         int32_t MB, int32_t NB, pkv_dtype cache_dtype, hipStream_t stream) {
  if (S < 0 || H <= 0 || D <= 0 || BS <= 0 || MB <= 0 || NB <= 0) return PKV_ERR_INVALID_ARG;
  if (!ok_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
  if (!ok_head_size(D) || !ok_block_size(BS)) return PKV_ERR_UNSUPPORTED;
  if (S > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  if (S == 0) return PKV_OK;
  if (!k_out || !v_out || !cu_lens || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_gather_kv(k_out, v_out, cu_lens, k_cache, v_cache, block_tables,
                                        context_lens, S, H, D, BS, MB, NB, cache_dtype, stream));
}

pkv_status pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes % 16 != 0) return PKV_ERR_INVALID_ARG;
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4)) return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_stream_read(buf, bytes, sink, stream));
}

}  // extern "C"

extern "C" {

size_t pkv_check_workspace_bytes(int32_t NB, int32_t BS) {
  if (NB <= 0 || BS <= 0) return 0;
  return pkv::check_layout(NB, BS).words * sizeof(uint32_t);
}

pkv_status pkv_check_step_inputs(const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t MB,
                                 const int32_t* slot_mapping, int32_t T, const int32_t* pairs, int32_t N,
                                 int32_t BS, int32_t NB, int32_t append, void* workspace,
                                 size_t workspace_bytes, uint32_t* violations, hipStream_t stream) {
  if (violations) *violations = 0;
  if (S < 0 || T < 0 || N < 0 || MB <= 0 || BS <= 0 || NB <= 0) return PKV_ERR_INVALID_ARG;
  if ((S > 0 && (!block_tables || !context_lens)) || (T > 0 && !slot_mapping) || (N > 0 && !pairs))
    return PKV_ERR_INVALID_ARG;
  if (append && T != S) return PKV_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 4)) return PKV_ERR_INVALID_ARG;
  if (workspace_bytes < pkv_check_workspace_bytes(NB, BS)) return PKV_ERR_WORKSPACE;
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  if (pkv::launch_check_step_inputs(block_tables, context_lens, S, MB, slot_mapping, T, pairs, N, BS, NB,
                                    append ? 1 : 0, ws, stream) != hipSuccess)
    return PKV_ERR_HIP;
  uint32_t mask = 0;
  if (hipMemcpyAsync(&mask, ws, sizeof(mask), hipMemcpyDeviceToHost, stream) != hipSuccess) return PKV_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PKV_ERR_HIP;
  if (violations) *violations = mask;
  return mask ? PKV_ERR_DEVICE_CHECK : PKV_OK;
}

}  // extern "C"

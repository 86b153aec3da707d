// Sanitizer run of the C ABI's host code (argument checks, dispatch,
// workspace arithmetic, graph set-up) with the kernel launchers stubbed out
// (launch_stubs.cpp), on a machine without a GPU.  Every call below either
// fails a host-side check, reaches a stub launcher, or reaches a HIP runtime
// call that fails for want of a device; the expected status of each is
// asserted.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host side; any report aborts the run.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "pagedkv.h"

extern int pkv_stub_launches;
extern int pkv_stub_static_lookups;

static int failures = 0;

static void expect(const char* what, int line, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect(#call, __LINE__, (int)(call), (int)(want))

// a call that passes every host check must reach exactly one more launcher
#define EXPECT_LAUNCH(call)                                   \
  do {                                                        \
    const int before_ = pkv_stub_launches;                    \
    EXPECT(call, PKV_OK);                                     \
    expect(#call " launches", __LINE__, pkv_stub_launches - before_ >= 1, 1); \
  } while (0)

int main() {
  // never dereferenced: the launchers are stubs
  void* f = reinterpret_cast<void*>(uintptr_t{0x100000});
  const int32_t* fi = static_cast<const int32_t*>(f);
  alignas(16) static unsigned char ws_host[1 << 16];
  void* ws = ws_host;

  EXPECT(pkv_version() >= 100, 1);
  for (int s : {0, 1, 2, 3, 4, 5, 6, 99}) EXPECT(pkv_status_string(static_cast<pkv_status>(s)) != nullptr, 1);
  EXPECT(pkv_reshape_and_cache(f, f, f, f, nullptr, 4, 1, 64, 16, 1, static_cast<pkv_dtype>(9), PKV_F32, 1.f, 1.f,
                               nullptr),
         PKV_ERR_INVALID_ARG);

  // cache write
  EXPECT_LAUNCH(pkv_reshape_and_cache(f, f, f, f, fi, 64, 40, 128, 16, 8951, PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr));
  EXPECT_LAUNCH(pkv_reshape_and_cache(f, f, f, f, fi, 256, 32, 128, 32, 12400, PKV_F16, PKV_FP8_E4M3, .05f, .07f,
                                      nullptr));
  EXPECT(pkv_reshape_and_cache(f, f, f, f, fi, 0, 1, 64, 16, 1, PKV_F32, PKV_F32, 1.f, 1.f, nullptr), PKV_OK);
  EXPECT(pkv_reshape_and_cache(f, f, f, f, fi, -1, 1, 64, 16, 1, PKV_F32, PKV_F32, 1.f, 1.f, nullptr),
         PKV_ERR_INVALID_ARG);
  EXPECT(pkv_reshape_and_cache(f, f, f, f, fi, 4, 1, 64, 16, 1, PKV_F32, PKV_F32, NAN, 1.f, nullptr),
         PKV_ERR_INVALID_ARG);
  EXPECT(pkv_reshape_and_cache(f, f, f, f, fi, 4, 1, 72, 16, 1, PKV_F32, PKV_F32, 1.f, 1.f, nullptr),
         PKV_ERR_UNSUPPORTED);

  // decode: workspace arithmetic at extreme sizes must not overflow
  EXPECT(pkv_decode_workspace_bytes(65535, 1024, 256, 16, 1 << 20) > 0, 1);
  EXPECT(pkv_decode_workspace_bytes(INT32_MAX, INT32_MAX, 256, 16, INT32_MAX) > 0, 1);
  EXPECT(pkv_decode_workspace_bytes(1, 1, 1, 1 << 30, INT32_MAX) >= 0, 1);
  const size_t need = pkv_decode_workspace_bytes(4, 2, 128, 16, 512);
  EXPECT(need > 0 && need <= sizeof(ws_host), 1);
  EXPECT_LAUNCH(pkv_paged_attention_decode(f, f, f, f, fi, fi, 64, 40, 128, 16, 128, 8951, .088f, PKV_BF16, PKV_BF16,
                                           1.f, 1.f, nullptr, 0, nullptr));
  EXPECT_LAUNCH(pkv_paged_attention_decode(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100, .088f, PKV_F16, PKV_F16, 1.f,
                                           1.f, ws, need, nullptr));
  EXPECT(pkv_paged_attention_decode(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100, .088f, PKV_F16, PKV_F16, 1.f, 1.f,
                                    ws, need - 1, nullptr),
         PKV_ERR_WORKSPACE);
  EXPECT(pkv_paged_attention_decode(f, f, f, f, fi, fi, 70000, 2, 128, 16, 8, 100, .088f, PKV_F16, PKV_F16, 1.f, 1.f,
                                    nullptr, 0, nullptr),
         PKV_ERR_UNSUPPORTED);
  // a table so long that the partitions would not fit the grid
  EXPECT(pkv_paged_attention_decode(f, f, f, f, fi, fi, 4, 2, 128, 16, INT32_MAX, 100, .088f, PKV_F16, PKV_F16, 1.f,
                                    1.f, ws, sizeof(ws_host), nullptr),
         PKV_ERR_UNSUPPORTED);
  EXPECT(pkv_paged_attention_decode_merge(f, fi, 4, 2, 128, 32, INT32_MAX, PKV_F16, PKV_F16, 1.f, ws,
                                          sizeof(ws_host), nullptr),
         PKV_ERR_UNSUPPORTED);
  EXPECT_LAUNCH(pkv_paged_attention_decode_partitions(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100, .088f, PKV_BF16,
                                                      PKV_INT8, .04f, .04f, ws, need, nullptr));
  EXPECT(pkv_paged_attention_decode_merge(f, fi, 4, 2, 128, 16, 512, PKV_BF16, PKV_INT8, .04f, ws, need, nullptr),
         PKV_OK);
  EXPECT_LAUNCH(pkv_paged_attention_decode_append(f, f, f, f, f, f, fi, fi, fi, 64, 40, 128, 16, 128, 8951, .088f,
                                                  PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr, 0, nullptr));
  EXPECT_LAUNCH(pkv_paged_attention_decode_append_partitions(f, f, f, f, f, f, fi, fi, fi, 4, 2, 96, 32, 300, 100,
                                                             .1f, PKV_F16, PKV_FP8_E4M3, .02f, .03f, ws, need,
                                                             nullptr));

  // the grouped decode: group sizes 1 .. 8, 16-bit / f32 pools only, the
  // new-token arguments all or none, an empty batch launches nothing
  EXPECT_LAUNCH(pkv_paged_attention_decode_grouped(f, f, f, f, f, f, fi, fi, fi, 64, 32, 128, 16, 49, 1010, .088f,
                                                   PKV_F16, PKV_F16, 8, nullptr, 0, nullptr));
  EXPECT_LAUNCH(pkv_paged_attention_decode_grouped_partitions(f, f, nullptr, nullptr, f, f, nullptr, fi, fi, 10, 3,
                                                              80, 32, 300, 100, .1f, PKV_BF16, PKV_BF16, 5, ws,
                                                              sizeof(ws_host), nullptr));
  for (int g : {0, 9, -1})
    EXPECT(pkv_paged_attention_decode_grouped(f, f, nullptr, nullptr, f, f, nullptr, fi, fi, 64, 32, 128, 16, 49,
                                              1010, .088f, PKV_F16, PKV_F16, g, nullptr, 0, nullptr),
           PKV_ERR_INVALID_ARG);
  EXPECT(pkv_paged_attention_decode_grouped(f, f, nullptr, nullptr, f, f, nullptr, fi, fi, 4, 2, 128, 32, 32, 100,
                                            .1f, PKV_F16, PKV_FP8_E4M3, 2, ws, need, nullptr),
         PKV_ERR_UNSUPPORTED);
  EXPECT(pkv_paged_attention_decode_grouped(f, f, f, nullptr, f, f, fi, fi, fi, 64, 32, 128, 16, 49, 1010, .088f,
                                            PKV_F16, PKV_F16, 8, nullptr, 0, nullptr),
         PKV_ERR_INVALID_ARG);
  {
    const int before = pkv_stub_launches;
    EXPECT(pkv_paged_attention_decode_grouped(f, f, nullptr, nullptr, f, f, nullptr, fi, fi, 0, 32, 128, 16, 49, 1010,
                                              .088f, PKV_F16, PKV_F16, 8, nullptr, 0, nullptr),
           PKV_OK);
    EXPECT(pkv_stub_launches - before, 0);
  }

  // the decode over the library's static workspace: the size limit and the
  // arguments are refused before the buffer is looked up or anything
  // launched; a call that needs no partials does not look it up either
  {
    const int lookups = pkv_stub_static_lookups;
    EXPECT(pkv_paged_attention_decode_static(f, f, f, f, fi, fi, 512, 64, 128, 16, 256, 100, .088f, PKV_BF16,
                                             PKV_BF16, 1.f, 1.f, nullptr),
           PKV_ERR_WORKSPACE);
    EXPECT(pkv_paged_attention_decode_static(f, f, f, f, fi, fi, -1, 64, 128, 16, 256, 100, .088f, PKV_BF16,
                                             PKV_BF16, 1.f, 1.f, nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT(pkv_paged_attention_decode_static(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100, NAN, PKV_F16, PKV_F16,
                                             1.f, 1.f, nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT(pkv_paged_attention_decode_static(f, f, f, f, fi, fi, 0, 2, 128, 16, 512, 100, .088f, PKV_F16, PKV_F16,
                                             1.f, 1.f, nullptr),
           PKV_OK);
    EXPECT(pkv_stub_static_lookups == lookups, 1);
    EXPECT_LAUNCH(pkv_paged_attention_decode_static(f, f, f, f, fi, fi, 64, 40, 128, 16, 128, 8951, .088f, PKV_BF16,
                                                    PKV_BF16, 1.f, 1.f, nullptr));
    EXPECT(pkv_stub_static_lookups == lookups, 1);
    // 256 x 32 heads over two partitions: 8.1 MiB of partials
    EXPECT_LAUNCH(pkv_paged_attention_decode_static(f, f, f, f, fi, fi, 256, 32, 128, 32, 128, 12400, .088f,
                                                    PKV_F16, PKV_FP8_E4M3, .05f, .05f, nullptr));
    EXPECT(pkv_stub_static_lookups == lookups + 1, 1);
  }

  // one scale per head: arrays required for 8-bit pools, ignored for 16-bit ones
  {
    const float* hs = reinterpret_cast<const float*>(f);
    const float* odd = reinterpret_cast<const float*>(uintptr_t{0x100002});   // not 4-byte aligned
    EXPECT_LAUNCH(pkv_reshape_and_cache_head_scales(f, f, f, f, fi, 256, 32, 128, 32, 12400, PKV_F16,
                                                    PKV_FP8_E4M3, hs, hs, nullptr));
    EXPECT(pkv_reshape_and_cache_head_scales(f, f, f, f, fi, 256, 32, 128, 32, 12400, PKV_F16, PKV_INT8, nullptr,
                                             hs, nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT(pkv_reshape_and_cache_head_scales(f, f, f, f, fi, 256, 32, 128, 32, 12400, PKV_F16, PKV_INT8, hs, odd,
                                             nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT_LAUNCH(pkv_reshape_and_cache_head_scales(f, f, f, f, fi, 64, 40, 128, 16, 8951, PKV_BF16, PKV_BF16,
                                                    nullptr, nullptr, nullptr));
    EXPECT_LAUNCH(pkv_paged_attention_decode_head_scales(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100, .088f,
                                                         PKV_F16, PKV_FP8_E4M3, hs, hs, ws, need, nullptr));
    EXPECT(pkv_paged_attention_decode_head_scales(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100, .088f, PKV_F16,
                                                  PKV_INT8, hs, nullptr, ws, need, nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT_LAUNCH(pkv_paged_attention_decode_partitions_head_scales(f, f, f, f, fi, fi, 4, 2, 128, 16, 512, 100,
                                                                    .088f, PKV_BF16, PKV_INT8, hs, hs, ws, need,
                                                                    nullptr));
    EXPECT(pkv_paged_attention_decode_merge_head_scales(f, fi, 4, 2, 128, 16, 512, PKV_BF16, PKV_INT8, hs, ws, need,
                                                        nullptr),
           PKV_OK);
    EXPECT(pkv_paged_attention_decode_merge_head_scales(f, fi, 4, 2, 128, 16, 512, PKV_BF16, PKV_INT8, nullptr, ws,
                                                        need, nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT_LAUNCH(pkv_paged_attention_decode_append_head_scales(f, f, f, f, f, f, fi, fi, fi, 4, 2, 96, 32, 300, 100,
                                                                .1f, PKV_F16, PKV_FP8_E4M3, hs, hs, ws, need,
                                                                nullptr));
    EXPECT_LAUNCH(pkv_paged_attention_decode_append_partitions_head_scales(
        f, f, f, f, f, f, fi, fi, fi, 64, 40, 128, 16, 128, 8951, .088f, PKV_BF16, PKV_BF16, nullptr, nullptr,
        nullptr, 0, nullptr));
    EXPECT_LAUNCH(pkv_paged_attention_prefill_head_scales(f, f, f, f, fi, fi, fi, 16, 28000, 2048, 40, 128, 16, 128,
                                                          2600, .088f, PKV_BF16, PKV_FP8_E4M3, hs, hs, nullptr));
    EXPECT(pkv_paged_attention_prefill_head_scales(f, f, f, f, fi, fi, fi, 16, 28000, 2048, 40, 128, 16, 128, 2600,
                                                   .088f, PKV_BF16, PKV_INT8, nullptr, nullptr, nullptr),
           PKV_ERR_INVALID_ARG);
    EXPECT_LAUNCH(pkv_paged_attention_prefill_append_head_scales(f, f, f, f, f, f, fi, fi, fi, fi, 5, 300, 100, 4,
                                                                 64, 16, 20, 64, .125f, PKV_F16, PKV_INT8, hs, hs,
                                                                 nullptr));
  }

  // prompt attention
  EXPECT_LAUNCH(pkv_paged_attention_prefill(f, f, f, f, fi, fi, fi, 16, 28000, 2048, 40, 128, 16, 128, 2600, .088f,
                                            PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr));
  EXPECT_LAUNCH(pkv_paged_attention_prefill_append(f, f, f, f, f, f, fi, fi, fi, fi, 5, 300, 100, 4, 64, 16, 20, 64,
                                                   .125f, PKV_F16, PKV_F16, 1.f, 1.f, nullptr));
  EXPECT(pkv_paged_attention_prefill(f, f, f, f, fi, fi, fi, 16, -1, 2048, 40, 128, 16, 128, 2600, .088f, PKV_BF16,
                                     PKV_BF16, 1.f, 1.f, nullptr),
         PKV_ERR_INVALID_ARG);
  EXPECT(pkv_paged_attention_prefill(f, f, f, f, fi, fi, fi, 16, 100, 2048, 40, 128, 16, 128, 2600, .088f, PKV_F32,
                                     PKV_F32, 1.f, 1.f, nullptr),
         PKV_ERR_UNSUPPORTED);
  // more heads than a grid dimension takes (and than the appending kernel's row offsets allow)
  EXPECT(pkv_paged_attention_prefill_append(f, f, f, f, f, f, fi, fi, fi, fi, 5, 300, 100, 65536, 64, 16, 20, 64,
                                            .125f, PKV_F16, PKV_F16, 1.f, 1.f, nullptr),
         PKV_ERR_UNSUPPORTED);

  // copies, gather, probe
  EXPECT_LAUNCH(pkv_copy_blocks(f, f, fi, 56, 32, 128, 16, 1010, PKV_F16, nullptr));
  EXPECT(pkv_copy_blocks(f, f, fi, 0, 32, 128, 16, 1010, PKV_F16, nullptr), PKV_OK);
  EXPECT_LAUNCH(pkv_gather_kv(f, f, fi, f, f, fi, fi, 4, 2, 64, 16, 8, 64, PKV_F32, nullptr));
  EXPECT_LAUNCH(pkv_stream_read(f, 1 << 20, static_cast<uint32_t*>(f), nullptr));
  // the swap resolves its pointers with the HIP runtime first: without a
  // device nothing resolves, and it refuses them
  EXPECT(pkv_swap_blocks(f, f, f, f, fi, 4, 2, 128, 16, 10, 10, PKV_F16, nullptr), PKV_ERR_INVALID_ARG);

  // device-side check: the launcher runs, reading the mask back needs a device
  uint32_t mask = 7;
  const size_t cneed = pkv_check_workspace_bytes(12400, 32);
  EXPECT(cneed > 0 && cneed <= sizeof(ws_host) * 2, 1);
  EXPECT(pkv_check_workspace_bytes(INT32_MAX, 32) > 0, 1);
  EXPECT(pkv_check_step_inputs(fi, fi, 4, 8, fi, 4, fi, 2, 16, 64, 1, ws, sizeof(ws_host), &mask, nullptr),
         PKV_ERR_HIP);
  EXPECT(mask, 0);
  EXPECT(pkv_check_step_inputs(fi, fi, 4, 8, fi, 3, fi, 2, 16, 64, 1, ws, sizeof(ws_host), &mask, nullptr),
         PKV_ERR_INVALID_ARG);

  // the decode graph: set-up fails at the device query and frees what it made
  pkv_decode_step step{};
  step.k_cache = step.v_cache = f;
  step.key = step.value = f;
  step.slot_mapping = fi;
  step.q = step.out = f;
  step.block_tables = step.context_lens = fi;
  step.S = 4; step.H = 2; step.D = 128; step.BS = 16; step.MB = 8; step.NB = 64;
  step.scale = .088f; step.k_scale = step.v_scale = 1.f;
  step.q_dtype = step.cache_dtype = PKV_F16;
  pkv_decode_graph* g = reinterpret_cast<pkv_decode_graph*>(f);
  EXPECT(pkv_decode_graph_create(&step, &g), PKV_ERR_HIP);
  EXPECT(g == nullptr, 1);
  step.S = 0;
  EXPECT(pkv_decode_graph_create(&step, &g), PKV_ERR_INVALID_ARG);
  EXPECT(pkv_decode_graph_create(nullptr, &g), PKV_ERR_INVALID_ARG);
  EXPECT(pkv_decode_graph_destroy(nullptr), PKV_OK);

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("abi host harness ok (%d launcher calls)\n", pkv_stub_launches);
  return 0;
}

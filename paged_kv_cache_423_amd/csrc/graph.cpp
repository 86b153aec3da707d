// HIP-graph capture of the decode step (declared in include/pagedkv.h).
//
// The l189.com article on KV cache and PagedAttention (www.l189.com/news/
// 180929) §3 captures the decode step once, over input buffers of a fixed
// maximum batch size, and replays the captured graph every step, which cuts
// the per-step launch overhead.  Here the step is: copy-on-write block
// copies, the cache write of one new token per batch slot, and the two
// phases of the decode (or, when the step asks for it, the decode that
// stores the step's tokens itself), all on the caller's fixed device buffers.  A replay
// re-reads every buffer, so the caller changes a step by rewriting their
// contents; batch slots without a sequence carry slot -1 (no write) and
// context length 0 (zero output), and unused copy pairs carry ids outside
// the pool (skipped).
//
// Capture runs on a private stream of default priority; nothing recorded
// into the graph is a memset.

#include <new>

#include "pagedkv.h"

struct pkv_decode_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int device = -1;
};

namespace {

pkv_status record_step(const pkv_decode_step* st, hipStream_t s) {
  pkv_status r = PKV_OK;
  // one scale per head when the step gives the arrays (8-bit pools)
  const bool head = st->k_scales || st->v_scales;
  if (st->num_pairs > 0) {
    r = pkv_copy_blocks(st->k_cache, st->v_cache, st->copy_pairs, st->num_pairs, st->H, st->D, st->BS, st->NB,
                        st->cache_dtype, s);
    if (r != PKV_OK) return r;
  }
  if (st->append) {
    // the decode stores the step's tokens itself (one kernel fewer)
    r = head ? pkv_paged_attention_decode_append_partitions_head_scales(
                   st->out, st->q, st->key, st->value, st->k_cache, st->v_cache, st->slot_mapping, st->block_tables,
                   st->context_lens, st->S, st->H, st->D, st->BS, st->MB, st->NB, st->scale, st->q_dtype,
                   st->cache_dtype, st->k_scales, st->v_scales, st->workspace, st->workspace_bytes, s)
             : pkv_paged_attention_decode_append_partitions(
                   st->out, st->q, st->key, st->value, st->k_cache, st->v_cache, st->slot_mapping, st->block_tables,
                   st->context_lens, st->S, st->H, st->D, st->BS, st->MB, st->NB, st->scale, st->q_dtype,
                   st->cache_dtype, st->k_scale, st->v_scale, st->workspace, st->workspace_bytes, s);
    if (r != PKV_OK) return r;
  } else {
    r = head ? pkv_reshape_and_cache_head_scales(st->key, st->value, st->k_cache, st->v_cache, st->slot_mapping,
                                                 st->S, st->H, st->D, st->BS, st->NB, st->q_dtype, st->cache_dtype,
                                                 st->k_scales, st->v_scales, s)
             : pkv_reshape_and_cache(st->key, st->value, st->k_cache, st->v_cache, st->slot_mapping, st->S, st->H,
                                     st->D, st->BS, st->NB, st->q_dtype, st->cache_dtype, st->k_scale, st->v_scale, s);
    if (r != PKV_OK) return r;
    r = head ? pkv_paged_attention_decode_partitions_head_scales(
                   st->out, st->q, st->k_cache, st->v_cache, st->block_tables, st->context_lens, st->S, st->H,
                   st->D, st->BS, st->MB, st->NB, st->scale, st->q_dtype, st->cache_dtype, st->k_scales,
                   st->v_scales, st->workspace, st->workspace_bytes, s)
             : pkv_paged_attention_decode_partitions(
                   st->out, st->q, st->k_cache, st->v_cache, st->block_tables, st->context_lens, st->S, st->H,
                   st->D, st->BS, st->MB, st->NB, st->scale, st->q_dtype, st->cache_dtype, st->k_scale,
                   st->v_scale, st->workspace, st->workspace_bytes, s);
    if (r != PKV_OK) return r;
  }
  return head ? pkv_paged_attention_decode_merge_head_scales(st->out, st->context_lens, st->S, st->H, st->D, st->BS,
                                                             st->MB, st->q_dtype, st->cache_dtype, st->v_scales,
                                                             st->workspace, st->workspace_bytes, s)
              : pkv_paged_attention_decode_merge(st->out, st->context_lens, st->S, st->H, st->D, st->BS, st->MB,
                                                 st->q_dtype, st->cache_dtype, st->v_scale, st->workspace,
                                                 st->workspace_bytes, s);
}

void release(pkv_decode_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // namespace

extern "C" {

pkv_status pkv_decode_graph_create(const pkv_decode_step* step, pkv_decode_graph** graph) {
  if (!graph) return PKV_ERR_INVALID_ARG;
  *graph = nullptr;
  if (!step || step->S <= 0 || step->num_pairs < 0) return PKV_ERR_INVALID_ARG;
  if (step->num_pairs > 0 && !step->copy_pairs) return PKV_ERR_INVALID_ARG;

  pkv_decode_graph* g = new (std::nothrow) pkv_decode_graph;
  if (!g) return PKV_ERR_HIP;
  if (hipGetDevice(&g->device) != hipSuccess) {
    release(g);
    return PKV_ERR_HIP;
  }
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
    release(g);
    return PKV_ERR_HIP;
  }
  pkv_status st = PKV_OK;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    st = PKV_ERR_HIP;
  } else {
    st = record_step(step, cs);
    hipGraph_t captured = nullptr;
    const hipError_t e = hipStreamEndCapture(cs, &captured);
    g->graph = captured;
    if (st == PKV_OK && (e != hipSuccess || !captured)) st = PKV_ERR_HIP;
  }
  if (st == PKV_OK && hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0) != hipSuccess) {
    g->exec = nullptr;
    st = PKV_ERR_HIP;
  }
  (void)hipStreamDestroy(cs);
  if (st != PKV_OK) {
    release(g);
    return st;
  }
  *graph = g;
  return PKV_OK;
}

pkv_status pkv_decode_graph_launch(pkv_decode_graph* graph, hipStream_t stream) {
  if (!graph || !graph->exec) return PKV_ERR_INVALID_ARG;
  return hipGraphLaunch(graph->exec, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_decode_graph_destroy(pkv_decode_graph* graph) {
  release(graph);
  return PKV_OK;
}

}  // extern "C"

#!/usr/bin/env python3
"""Decode-step benchmark: paged-attention decode K/V-read GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one pass of the whole hot path over one batch: the copy-on-write
block copies (only the shared-prefix workload has any), then the cache write
of one new token per sequence and the decode, done by
paged_attention_decode_append: its partition kernel takes each sequence's
new token as the row at position n - 1 and stores it at its slot, and the
partition merge runs when a context spans several partitions.  The same step
with the cache write as a kernel of its own (reshape_and_cache, then
paged_attention_decode) is timed too, as ``unfused_ms_per_step``.  Each call
of the step is prepared once before the loops (the binding's
``prepare=True``: arguments checked and marshalled once, as a serving loop
over fixed batch buffers would); every step launches all of its kernels.
Inputs are seeded synthetic tensors already resident in HBM.  The default workload is
the Llama2-13B-shaped long-context decode: 64 sequences x 40 heads x 128,
block size 16, bf16, context lengths U[1536, 2048].

Printed: one JSON line.  ``value`` is K/V bytes read per step (sum over
sequences of n_s * H * D * 2 * element size) divided by the wall time per
step, over a timed loop without timing events.  ``roofline`` rates the
decode's partition kernel against 8 TB/s HBM with its duration measured by
HIP events on the launch stream around 20 back-to-back launches queued
behind GPU work (so that the small workloads, whose steps the host's launch
pace bounds, time the kernel and not the enqueue gaps).  A second pass of
the same steps records events on every fourth step (an event record costs
the GPU a few microseconds) for the in-step phase times reported beside it.
With shared prefixes the roofline counts each physical K/V row once.  ``stream_read`` is the
library's read-only probe over a 4 GiB buffer, the device's achievable
sequential read rate with the same loads; ``roofline.frac_of_stream_read``
rates the partition kernel against it.
``cpu_baseline`` is the oracle (fp64 NumPy) timed on this host's cores on a
bounded sample of the same workload, as a reference point only.
``components`` times the step's cache write and (where the workload has
them) its copy-on-write block copies on their own, each as GB/s of its own
bytes; ``pool`` gives the block pool's use after the step (blocks holding
tokens, and the share of their slots left empty).

``--prefill N`` measures a prompt step instead (the prompt attention that
also stores the prompt's K/V; TFLOP/s of 4 * D flops per visible (query,
key) pair and head): ``roofline`` rates that step's kernels, and
``attention_only_roofline`` the attention alone, against the 2.5 PFLOP/s
dense 16-bit MFMA peak, both from back-to-back launches queued behind GPU
work as above; ``prefill_ms`` is the in-step event time.
"""

from __future__ import annotations

import argparse
import contextlib
import gc
import json
import math
import multiprocessing as mp
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402


@contextlib.contextmanager
def _no_gc():
    """A timed region without Python's garbage collector: a full collection
    over the workload generator's many small objects can stall the host for
    tens of milliseconds, and a stall while the device's queue is empty (the
    first steps after a synchronise) shows up in the GPU's own timestamps."""
    gc.collect()
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
EVENT_STRIDE = 4                # timing events on every 4th timed step
WORKLOAD_NAMES = {
    1: "tiny fp32 decode: 4 seqs x 4 heads x 64, block 16, ctx U[1,100]",
    2: "LLaMA-7B-shaped layer, fp16 KV: 16 seqs x 32 heads x 128, block 16, ctx U[50,178]",
    3: "Llama2-13B-shaped long-context decode, bf16 KV: 64 seqs x 40 heads x 128, block 16, ctx U[1536,2048]",
    4: "shared-prefix copy-on-write, fp16 KV: 8 groups x 8 seqs x 32 heads x 128, 512-token prefix + U[1,256] tails",
    5: "fp8-e4m3 KV, fp16 q/out: 256 seqs x 32 heads x 128, block 32, ctx log-U[128,4096]",
    6: "int8 KV, fp16 q/out: 256 seqs x 32 heads x 128, block 32, ctx log-U[128,4096]",
}

def decode_config(index: int, head_scales: bool = False):
    """Decode workload ``index``; with head_scales, its 8-bit pools carry one
    scale per head (workloads 5 and 6)."""
    import workloads as W
    if not head_scales:
        return W.CONFIGS[index]
    per_head = {5: W.CONFIG_5_HEAD_SCALES, 6: W.CONFIG_6_HEAD_SCALES}
    if index not in per_head:
        raise SystemExit("--head-scales applies to the 8-bit workloads (--config 5 or 6)")
    return per_head[index]


# ------------------------------------------------------------------ CPU baseline (oracle)

_SAMPLE = {}


def _oracle_chunk(seqs):
    import oracle
    c = _SAMPLE
    oracle.paged_attention_decode(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["scale"], c["qd"], c["cd"],
                                  c["ks"], c["vs"], seqs=seqs)
    return len(seqs)


def _timed_passes(fn, chunks, cores: int, min_seconds: float):
    """Whole passes of fn over chunks in ``cores`` fork workers until
    min_seconds of wall time; returns (passes, seconds).  The pool is closed
    and its workers joined before returning, so none outlives the run."""
    ctx = mp.get_context("fork")
    pool = ctx.Pool(cores)
    try:
        pool.map(fn, [chunks[0][:1]] * cores)               # workers up and warm
        passes = 0
        t0 = time.perf_counter()
        while True:
            pool.map(fn, chunks)
            passes += 1
            wall = time.perf_counter() - t0
            if wall >= min_seconds:
                break
    finally:
        pool.close()
        pool.join()
    return passes, wall


def cpu_baseline(cfg_index: int, sample_seqs: int, min_seconds: float = 10.0, head_scales: bool = False):
    """Time the oracle's decode on a sample of the workload on this host's cores:
    whole passes over ``sample_seqs`` sequences (all heads), repeated until
    ``min_seconds`` of wall time have been spent.

    Runs before anything touches the GPU, so the worker processes are forked
    from a process without a GPU context."""
    import workloads as W
    cfg = decode_config(cfg_index, head_scales)
    case = W.make_case(cfg, device="cpu", S=min(sample_seqs, cfg.S))
    _SAMPLE.update(q=W.bits(case.q, cfg.q_dtype), k=W.bits(case.k_cache, cfg.cache_dtype),
                   v=W.bits(case.v_cache, cfg.cache_dtype), tables=case.block_tables, lens=case.context_lens,
                   scale=case.scale, qd=cfg.q_dtype, cd=cfg.cache_dtype, ks=case.k_scale, vs=case.v_scale)
    cores = min(len(os.sched_getaffinity(0)), 16, case.S)
    chunks = [list(c) for c in np.array_split(np.arange(case.S), cores) if len(c)]
    passes, wall = _timed_passes(_oracle_chunk, chunks, cores, min_seconds)
    kvb = case.kv_bytes * passes
    return {
        "value": round(kvb / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{passes} passes of the decode of {case.S} of the workload's {cfg.S} sequences (all "
                   f"{case.H} heads, {case.kv_bytes / 1e9:.3f} GB of K/V per pass): fp64 NumPy gather + softmax "
                   f"attention, {cores} worker processes, {wall:.2f} s wall; cache write not included"),
        "seconds": round(wall, 3),
        "seq_heads_per_s": round(passes * case.S * case.H / wall, 2),
    }


# ------------------------------------------------------------------ HBM traffic record

TRAFFIC_RECORDS = {3: "paged_decode_kernel.llama2-13b-longctx-bf16.hbm_traffic.md",
                   4: "paged_decode_kernel.shared-prefix-cow-f16.hbm_traffic.md",
                   5: "paged_decode_kernel.fp8-e4m3-kv.hbm_traffic.md",
                   6: "paged_decode_kernel.int8-kv.hbm_traffic.md"}
# the grouped decode's records, by (workload, group size)
GROUPED_TRAFFIC_RECORDS = {(4, 8): "paged_decode_group_kernel.shared-prefix-cow-f16.hbm_traffic.md"}
DECODE_SOURCES = ("attention.hip", "device_common.h", "kernels.h")


def decode_source_digest() -> str:
    """sha256 over the decode kernel's sources and build flags (include
    directories as paths relative to the repository, so that the digest does
    not depend on where the checkout sits)."""
    import hashlib
    from paged_kv_cache_423_amd import build as B
    flags = [("-I" + os.path.relpath(f[2:], ROOT)) if f.startswith("-I") else f for f in B.common_flags()]
    h = hashlib.sha256(" ".join(flags).encode())
    for name in DECODE_SOURCES:
        with open(os.path.join(B.CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(cfg_index: int, group_size: int = 1):
    """HBM bytes per partition-kernel launch from the committed counter
    record (read counter scaled by the copy calibration, plus the write
    counter), or None when there is no record or the kernel's sources have
    changed since the counters were taken.  group_size > 1: the grouped
    decode's record for that group size."""
    name = (TRAFFIC_RECORDS.get(cfg_index) if group_size <= 1
            else GROUPED_TRAFFIC_RECORDS.get((cfg_index, group_size)))
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("record: "):
                rec = json.loads(line[len("record: "):])
    if rec.get("source_digest") != decode_source_digest():
        return None
    return int(rec["traffic_bytes_per_launch"])


# ------------------------------------------------------------------ GPU

def gpu_bench(cfg_index: int, steps: int, warmup: int, cold_iters: int, graph: bool = False,
              head_scales: bool = False, group_size: int = 1):
    import torch
    import paged_kv_cache_423_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    pkv.lib()                                        # no fallback: raises if the library is missing
    cfg = decode_config(cfg_index, head_scales)
    case = W.make_case(cfg, device="cuda")
    dev = "cuda"
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    pairs = torch.from_numpy(case.copy_pairs).to(dev) if case.copy_pairs.shape[0] else None
    out = torch.empty_like(case.q)
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
    # one scale per head: float32 [H] device tensors, moved once, outside every timed region
    ks, vs = case.k_scale, case.v_scale
    if np.ndim(ks):
        ks, vs = torch.from_numpy(np.asarray(ks)).to(dev), torch.from_numpy(np.asarray(vs)).to(dev)
    torch.cuda.synchronize()

    # Timing events go on every EVENT_STRIDE-th step only: each event record
    # costs the GPU a few microseconds of its own (about 2% of a long-context
    # step with events on every step), which the other steps are spared.
    timed = [i for i in range(steps) if i % EVENT_STRIDE == 0]
    ev = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for i in timed}

    # Every call of the step is prepared once (arguments checked and
    # marshalled before the loops, as a serving loop over fixed batch
    # buffers would); each step then launches the same kernels again.
    if group_size > 1:
        # groups of group_size consecutive sequences read the blocks they
        # all map once; the grouped kernel also stores the step's tokens
        partitions = pkv.paged_attention_decode_grouped_partitions(
            out, case.q, case.k_cache, case.v_cache, bt, cl, case.scale, group_size, key=case.key,
            value=case.value, slot_mapping=slots, workspace=ws, prepare=True)
    else:
        partitions = pkv.paged_attention_decode_append_partitions(
            out, case.q, case.key, case.value, case.k_cache, case.v_cache, slots, bt, cl, case.scale, ks, vs,
            workspace=ws, prepare=True)
    merge = pkv.paged_attention_decode_merge(out, cl, case.BS, case.MB, case.k_cache.dtype, vs, workspace=ws,
                                             prepare=True)
    copies = pkv.copy_blocks(case.k_cache, case.v_cache, pairs, prepare=True) if pairs is not None else None
    write = pkv.reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache, slots, ks, vs, prepare=True)
    if group_size > 1:
        plain_partitions = pkv.paged_attention_decode_grouped_partitions(
            out, case.q, case.k_cache, case.v_cache, bt, cl, case.scale, group_size, workspace=ws, prepare=True)
    else:
        plain_partitions = pkv.paged_attention_decode_partitions(out, case.q, case.k_cache, case.v_cache, bt, cl,
                                                                 case.scale, ks, vs, workspace=ws, prepare=True)

    def step(e=None):
        # block copies (copy-on-write), then the decode that also writes the
        # step's new tokens, run as its two phases so that its partition
        # kernel is timed on its own; together they are exactly
        # paged_attention_decode_append
        if copies is not None:
            copies()
        if e is not None:
            e[0].record()
        partitions()
        if e is not None:
            e[1].record()
        merge()
        if e is not None:
            e[2].record()

    def unfused_step(e=None):
        # the same step with the cache write as a kernel of its own (events
        # at the same places, so that both loops carry the same instrumentation)
        if copies is not None:
            copies()
        if e is not None:
            e[0].record()
        write()
        plain_partitions()
        if e is not None:
            e[1].record()
        merge()
        if e is not None:
            e[2].record()

    def timed_loop(fn, with_events=True):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        with _no_gc():
            t0 = time.perf_counter()
            for i in range(steps):
                fn(ev.get(i) if with_events else None)
            torch.cuda.synchronize()
            return time.perf_counter() - t0

    # the timed step carries no events (the line's value); a second pass of
    # the same steps carries them on every EVENT_STRIDE-th step, for the
    # phase breakdown
    wall = timed_loop(step, False)
    instrumented_wall = timed_loop(step)
    decode_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in timed]
    part_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in timed]
    # the step with a separate cache-write kernel, for comparison
    unfused_wall = timed_loop(unfused_step, False)
    graphs = None
    if graph:
        # the step four ways, each without timing events, same run: eager
        # calls with the cache write as its own kernel or inside the decode,
        # and the same two forms captured once as a HIP graph and replayed
        graphs = {"eager_separate_write_ms": timed_loop(unfused_step, False) / steps * 1e3,
                  "eager_appending_decode_ms": timed_loop(step, False) / steps * 1e3}
        for name, append in (("graph_separate_write_ms", False), ("graph_appending_decode_ms", True)):
            g = pkv.DecodeGraph(case.k_cache, case.v_cache, case.key, case.value, slots, case.q, out, bt, cl,
                                case.scale, ks, vs, copy_pairs=pairs, workspace=ws, append=append)
            graphs[name] = timed_loop(lambda e=None: g.launch(), False) / steps * 1e3
            g.destroy()
        graphs = {k: round(v, 5) for k, v in graphs.items()}

    # Kernels timed on their own, back to back on the device: each call
    # takes less GPU time than (or, for the small workloads, about as much as)
    # the host needs to enqueue it, so the GPU is first kept busy with fills
    # of a 1 GiB buffer while the host queues COMPONENT_REPS calls, and one
    # event pair brackets those calls alone.  Median per call over
    # COMPONENT_ROUNDS rounds.  This is the partition kernel's duration the
    # roofline uses (the in-loop events of a host-bound step time the host's
    # enqueue gaps too), and it times the step's cache write and copies.
    busy = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def time_each(fn):
        return queued_launch_ms(fn, busy)

    # the step's partition kernel: for 8-bit pools the appending form runs the
    # cache-write kernel first, so the kernel is timed through the plain
    # partitions call, which launches the same partition kernel alone
    if case.cache_dtype in W.SCALED_FORMATS:
        kernel_ms = time_each(lambda: pkv.paged_attention_decode_partitions(
            out, case.q, case.k_cache, case.v_cache, bt, cl, case.scale, ks, vs, workspace=ws))
    else:
        kernel_ms = time_each(partitions)
    parts = {"reshape_and_cache_ms": time_each(lambda: pkv.reshape_and_cache(
        case.key, case.value, case.k_cache, case.v_cache, slots, ks, vs))}
    if pairs is not None:
        parts["copy_blocks_ms"] = time_each(lambda: pkv.copy_blocks(case.k_cache, case.v_cache, pairs))
    del busy

    # cold-cache decode: overwrite a 1 GiB buffer (more than the 256 MB
    # last-level cache plus all L2s) before each timed decode
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(cold_iters):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pkv.paged_attention_decode(out, case.q, case.k_cache, case.v_cache, bt, cl, case.scale, ks, vs, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    return (case, wall, instrumented_wall, decode_ms, part_ms, kernel_ms, unfused_wall, cold, graphs,
            stream_read_bench(), parts)


def pool_report(case):
    """Block-pool use after the step, as a serving system would monitor it:
    physical blocks holding tokens against the pool's blocks, and internal
    fragmentation, the share of those blocks' slots that hold no token
    (a shared block counts once)."""
    held = set()
    for s in range(case.S):
        n = int(case.context_lens[s])
        for t in range(n):
            held.add((int(case.block_tables[s, t // case.BS]), t % case.BS))
    blocks = {b for b, _ in held}
    return {"num_blocks": case.NB, "blocks_in_use": len(blocks),
            "utilisation": round(len(blocks) / case.NB, 4),
            "internal_fragmentation": round(1 - len(held) / max(1, len(blocks) * case.BS), 4)}


COMPONENT_REPS = 20
COMPONENT_ROUNDS = 5
BUSY_FILLS = 6              # 1 GiB fills queued ahead of the calls (about 1.2 ms of GPU work)


def queued_launch_ms(fn, busy):
    """Device time per call of ``fn``: COMPONENT_REPS calls queued back to
    back behind BUSY_FILLS fills of ``busy`` (so that the GPU, not the
    host's enqueue pace, sets the pace), one HIP event pair around the calls
    alone on torch's current stream, the median per call over
    COMPONENT_ROUNDS rounds."""
    import torch
    for _ in range(5):
        fn()
    per_call = []
    with _no_gc():
        for _ in range(COMPONENT_ROUNDS):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for v in range(BUSY_FILLS):
                busy.fill_(v)
            a.record()
            for _ in range(COMPONENT_REPS):
                fn()
            b.record()
            torch.cuda.synchronize()
            per_call.append(a.elapsed_time(b) / COMPONENT_REPS)
    return statistics.median(per_call)


def component_report(case, parts):
    """The cache write and the block copies timed on their own, each as GB/s
    of its own bytes: the write reads the new tokens' K/V and writes them
    into the pools (T * H * D * (source + cache element) * 2 for K and V);
    a copy reads and writes both pools' whole blocks
    (N * 2 * H * BS * D * element * 2)."""
    import workloads as W
    T, H, D = case.S, case.H, case.D
    src_b = W.ELEM_BYTES[case.q_dtype]
    cache_b = W.ELEM_BYTES[case.cache_dtype]
    wb = T * H * D * (src_b + cache_b) * 2
    ms = parts["reshape_and_cache_ms"]
    rep = {"reshape_and_cache": {"ms_per_call": round(ms, 5), "bytes": wb, "GBps": round(wb / (ms / 1e3) / 1e9, 1),
                                 "tokens": T}}
    if "copy_blocks_ms" in parts:
        n = int(case.copy_pairs.shape[0])
        cb = n * 2 * H * case.BS * D * cache_b * 2
        ms = parts["copy_blocks_ms"]
        rep["copy_blocks"] = {"ms_per_call": round(ms, 5), "bytes": cb, "GBps": round(cb / (ms / 1e3) / 1e9, 1),
                              "pairs": n}
    rep["timing"] = (f"one HIP event pair around {COMPONENT_REPS} back-to-back calls queued behind "
                     f"{BUSY_FILLS} GiB of fills, per call, median of {COMPONENT_ROUNDS} rounds")
    return rep


STREAM_BYTES = 4 << 30


def stream_read_bench(nbytes: int = STREAM_BYTES, launches: int = 10):
    """The library's read-only probe over a 4 GiB device buffer: the device's
    achievable sequential read rate with the decode's own 16-byte
    non-temporal loads, a second denominator beside the published peak."""
    import torch
    import paged_kv_cache_423_amd as pkv
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pkv.stream_read(buf, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in evs:
        a.record()
        pkv.stream_read(buf, sink)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.fmean(a.elapsed_time(b) for a, b in evs)
    del buf
    return {"GBps": round(nbytes / (ms / 1e3) / 1e9, 1), "bytes": nbytes, "launches": launches,
            "kernel": "stream_read_kernel: each 16-byte chunk read once, non-temporal; contiguous 8 KiB spans per wave"}


def calibrate_copy(passes: int = 3):
    """A plain copy of known size through copy_blocks, for scaling the HBM
    byte counters: 4096 whole blocks of a [8192, 40, 16, 128] bf16 pool pair
    (671 MB per pool), read once and written once per pass."""
    import torch
    import paged_kv_cache_423_amd as pkv
    torch.cuda.set_device(0)
    pkv.lib()
    NB, H, BS, D, N = 8192, 40, 16, 128, 4096
    k = torch.ones((NB, H, BS, D), dtype=torch.bfloat16, device="cuda")
    v = torch.ones_like(k)
    pairs = torch.stack([torch.arange(N), torch.arange(N, 2 * N)], 1).to(torch.int32).cuda()
    block_bytes = H * BS * D * 2
    for _ in range(passes):
        pkv.copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    return {"calibration": "copy_blocks", "passes": passes, "pairs": N,
            "bytes_read_per_launch": 2 * N * block_bytes, "bytes_written_per_launch": 2 * N * block_bytes}


# ------------------------------------------------------------------ prompt (multi-query) step

MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 matrix peak
PREFILL_NAMES = {
    1: "tiny prompts, fp16: 5 seqs x 4 heads x 64, block 16, new U[1,100] after cached U[0,40]",
    2: "LLaMA-7B-shaped prompts, fp16: 16 seqs x 32 heads x 128, block 16, prompts U[40,60]",
    3: "Llama2-13B-shaped long prompts, bf16: 16 seqs x 40 heads x 128, block 16, prompts U[1536,2048]",
    4: "shared-prefix prompts, fp16: 8 groups x 8 seqs x 32 heads x 128, cached 512-token prefix + U[1,256] new",
}
_PSAMPLE = {}


def _oracle_prefill_chunk(seqs):
    import oracle
    c = _PSAMPLE
    rows = []
    for s in seqs:
        a, b = int(c["cu"][s]), int(c["cu"][s + 1])
        oracle.paged_attention_prefill_seq(c["q"][a:b], c["k"], c["v"], c["tables"][s], int(c["lens"][s]), c["scale"],
                                           c["dt"], c["cdt"], c["ks"], c["vs"])
        rows.append(b - a)
    return sum(rows)


def prefill_config(index: int, cache: str = ""):
    """Prompt workload ``index``, with its pools in ``cache`` format (e4m3 /
    i8, per-pool scales) when given."""
    from dataclasses import replace
    import workloads as W
    cfg = W.PREFILL_CONFIGS[index]
    return replace(cfg, cache_dtype=cache) if cache else cfg


def prefill_cpu_baseline(cfg, min_seconds: float = 10.0):
    """The oracle's prompt attention on this host's cores, whole passes over
    the workload's sequences (at most 8 of them) until ``min_seconds`` of
    wall time; reported in TFLOP/s on the same flop count as the GPU."""
    import workloads as W
    case = W.make_prefill_case(cfg, device="cpu", S=min(8, cfg.S))
    dt, cdt = cfg.dtype, case.pool_dtype
    # the attention reads the cache as it is after the step's write (not timed)
    import oracle
    kb, vb = oracle.reshape_and_cache(W.bits(case.key, dt), W.bits(case.value, dt), W.bits(case.k_cache, cdt),
                                      W.bits(case.v_cache, cdt), case.slot_mapping, dt, cdt, case.k_scale,
                                      case.v_scale)
    _PSAMPLE.update(q=W.bits(case.q, dt), k=kb, v=vb, tables=case.block_tables, lens=case.context_lens,
                    cu=case.cu_q_lens, scale=case.scale, dt=dt, cdt=cdt, ks=case.k_scale, vs=case.v_scale)
    cores = min(len(os.sched_getaffinity(0)), 16, case.S)
    order = np.argsort(-case.q_lens.astype(np.int64))
    chunks = [list(map(int, order[i::cores])) for i in range(cores)]
    passes, wall = _timed_passes(_oracle_prefill_chunk, chunks, cores, min_seconds)
    flops = case.flops * passes
    return {
        "value": round(flops / wall / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{passes} passes of the prompt attention of {case.S} of the workload's {cfg.S} sequences "
                   f"({case.Tq} new tokens, {case.H} heads, {case.flops / 1e9:.2f} GFLOP per pass): fp64 NumPy "
                   f"gather + masked softmax attention, {cores} worker processes, {wall:.2f} s wall"),
        "seconds": round(wall, 3),
    }


def prefill_gpu_bench(cfg, steps: int, warmup: int):
    import torch
    import paged_kv_cache_423_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    pkv.lib()
    case = W.make_prefill_case(cfg, device="cuda")
    ks, vs = case.k_scale, case.v_scale
    dev = "cuda"
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    cu = torch.from_numpy(case.cu_q_lens).to(dev)
    pairs = torch.from_numpy(case.copy_pairs).to(dev) if case.copy_pairs.shape[0] else None
    out = torch.empty_like(case.q)
    torch.cuda.synchronize()
    timed = [i for i in range(steps) if i % EVENT_STRIDE == 0]     # steps that carry timing events
    ev = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for i in timed}

    # every call of the step prepared once before the loops (as in the decode bench)
    copies = pkv.copy_blocks(case.k_cache, case.v_cache, pairs, prepare=True) if pairs is not None else None
    fused = pkv.paged_attention_prefill_append(out, case.q, case.key, case.value, case.k_cache, case.v_cache, slots,
                                               bt, cl, cu, case.max_q_len, case.scale, ks, vs, prepare=True)
    write = pkv.reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache, slots, ks, vs, prepare=True)
    attend = pkv.paged_attention_prefill(out, case.q, case.k_cache, case.v_cache, bt, cl, cu, case.max_q_len,
                                         case.scale, ks, vs, prepare=True)

    def step(e=None):
        # block copies (copy-on-write), then the prompt attention that also
        # stores the new tokens' K/V (paged_attention_prefill_append)
        if copies is not None:
            copies()
        if e is not None:
            e[0].record()
        fused()
        if e is not None:
            e[1].record()

    def unfused_step(e=None):
        # the same step with the cache write as a kernel of its own
        if copies is not None:
            copies()
        if e is not None:
            e[0].record()
        write()
        if e is not None:
            e[1].record()
        attend()
        if e is not None:
            e[2].record()

    def timed_loop(fn, with_events=True):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        with _no_gc():
            t0 = time.perf_counter()
            for i in range(steps):
                fn(ev.get(i) if with_events else None)
            torch.cuda.synchronize()
            return time.perf_counter() - t0

    # timed loops without events (the line's value and the unfused step), then
    # the same steps again with events on every EVENT_STRIDE-th step for the
    # kernel times
    wall = timed_loop(step, False)
    timed_loop(step)
    attn_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in timed]
    assert torch.isfinite(out.float()).all(), "non-finite prompt attention output"
    unfused_wall = timed_loop(unfused_step, False)
    timed_loop(unfused_step)
    write_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in timed]
    unfused_attn_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in timed]
    # the kernels' own durations, launched back to back behind GPU work (the
    # in-step events of the small, host-bound workloads time enqueue gaps too)
    busy = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    queued = {"fused": queued_launch_ms(fused, busy), "attention": queued_launch_ms(attend, busy)}
    del busy
    return case, wall, attn_ms, write_ms, unfused_wall, unfused_attn_ms, queued


def prefill_main(a) -> int:
    cfg = prefill_config(a.prefill, a.prefill_cache)
    cpu = None if a.no_cpu_baseline else prefill_cpu_baseline(cfg, a.cpu_seconds)
    case, wall, attn_ms, write_ms, unfused_wall, unfused_attn_ms, queued = prefill_gpu_bench(cfg, a.steps, a.warmup)
    ms_step = wall / a.steps * 1e3
    attn = statistics.fmean(attn_ms)
    achieved = case.flops / (queued["fused"] / 1e3) / 1e12
    attn_only = case.flops / (queued["attention"] / 1e3) / 1e12
    q = np.percentile(attn_ms, [10, 50, 90])
    line = {
        "metric": "paged-attn prefill TFLOP/s (% of MFMA peak) and new tokens/s",
        "value": round(case.flops / (ms_step / 1e3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype if not case.cache_dtype else f"{case.dtype} / {case.cache_dtype} KV",
        "data": "synthetic",
        "config": {"workload": PREFILL_NAMES[a.prefill] + (f", {case.cache_dtype} pools" if case.cache_dtype else ""),
                   "num_seqs": case.S, "num_heads": case.H,
                   "head_size": case.D, "block_size": case.BS, "new_tokens": case.Tq,
                   "context_tokens": int(case.context_lens.sum()), "attended_pairs_per_head": case.attn_pairs,
                   "flops_per_step": case.flops},
        "new_tokens_per_s": round(case.Tq / (ms_step / 1e3), 1),
        "prefill_ms": {"mean": round(attn, 4), "p10": round(float(q[0]), 4), "p50": round(float(q[1]), 4),
                       "p90": round(float(q[2]), 4)},
        "step_mode": "calls prepared once before the loop, cache write fused into the prompt attention, no "
                     "timing events in the timed loop (prefill_ms: a second pass of the same steps with events on "
                     f"every {EVENT_STRIDE}th step)",
        "unfused_ms_per_step": round(unfused_wall / a.steps * 1e3, 4),
        "unfused_prefill_ms_mean": round(statistics.fmean(unfused_attn_ms), 4),
        "reshape_and_cache_ms_mean": round(statistics.fmean(write_ms), 5),
        # the attention alone (the unfused step's prompt kernel) against the same peak
        "attention_only_roofline": {"kernel": "paged_prefill_kernel", "duration_ms": round(queued["attention"], 5),
                                    "achieved": round(attn_only, 2),
                                    "frac": round(attn_only / MFMA_PEAK_TFLOPS, 4)},
        "roofline": {"bound": "mfma",
                     "kernel": ("reshape_and_cache_kernel then paged_prefill_kernel (8-bit pools: the cache write "
                                "quantises first)" if case.cache_dtype
                                else "paged_prefill_kernel (storing the new tokens' K/V too)"),
                     "duration": f"{COMPONENT_REPS} back-to-back launches queued behind GPU work, median of "
                                 f"{COMPONENT_ROUNDS} rounds",
                     "duration_ms": round(queued["fused"], 5),
                     "achieved": round(achieved, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


# ------------------------------------------------------------------ swap space (host <-> GPU blocks)

def swap_main(a) -> int:
    """Swap-out and swap-in of whole blocks between Llama2-13B-shaped bf16
    pools ([NB, 40, 16, 128], 163,840 B per block and pool) and a swap space
    in pinned host memory, next to a plain DMA copy of the same bytes."""
    import torch
    import paged_kv_cache_423_amd as pkv
    torch.cuda.set_device(0)
    pkv.lib()
    NB, H, BS, D, N = 8192, 40, 16, 128, 2048
    gen = torch.Generator(device="cuda").manual_seed(423)
    gk = torch.randn((NB, H, BS, D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gv = torch.randn((NB, H, BS, D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    hk = torch.empty((N, H, BS, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(7))[:N].to(torch.int32)
    out_pairs = torch.stack([perm, torch.arange(N, dtype=torch.int32)], 1).cuda()
    in_pairs = torch.stack([torch.arange(N, dtype=torch.int32), perm.flip(0)], 1).cuda()
    nbytes = 2 * N * H * BS * D * 2

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with _no_gc():
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out_ms = timed(lambda: pkv.swap_blocks(hk, hv, gk, gv, out_pairs), a.steps)
    in_ms = timed(lambda: pkv.swap_blocks(gk, gv, hk, hv, in_pairs), a.steps)
    dk = torch.empty((N, H, BS, D), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    dma_out_ms = timed(lambda: (hk.copy_(dk, non_blocking=True), hv.copy_(dv, non_blocking=True)), a.steps)
    dma_in_ms = timed(lambda: (dk.copy_(hk, non_blocking=True), dv.copy_(hv, non_blocking=True)), a.steps)
    gbps = lambda ms: round(nbytes / (ms / 1e3) / 1e9, 2)
    line = {
        "metric": "paged KV block swap GB/s (GPU pools <-> pinned host swap space)",
        "value": gbps((out_ms + in_ms) / 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": 2,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap of 2048 randomly placed Llama2-13B-shaped blocks (40 heads x 16 x 128, bf16) "
                               "out to pinned host memory and back", "blocks": N,
                   "bytes_per_direction": nbytes},
        "swap_out_ms": round(out_ms, 4), "swap_out_GBps": gbps(out_ms),
        "swap_in_ms": round(in_ms, 4), "swap_in_GBps": gbps(in_ms),
        "dma_copy_reference": {"d2h_GBps": gbps(dma_out_ms), "h2d_GBps": gbps(dma_in_ms),
                               "what": "torch copy_ of one contiguous pinned buffer of the same bytes (K and V)"},
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=3, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--cold-iters", type=int, default=10)
    ap.add_argument("--cpu-sample-seqs", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--head-scales", action="store_true",
                    help="with --config 5 or 6: one scale per head of the 8-bit pools instead of one per pool")
    ap.add_argument("--group-size", type=int, default=1,
                    help="decode groups of this many consecutive sequences that read the blocks they all map once "
                         "(2-8; the shared-prefix workload has groups of 8)")
    ap.add_argument("--graph", action="store_true",
                    help="time the decode step as a replay of its HIP graph; graph_comparison gives the step "
                         "eager and as a graph, with the cache write separate and inside the decode")
    ap.add_argument("--swap", action="store_true",
                    help="time block swaps between the GPU pools and a pinned host swap space")
    ap.add_argument("--prefill", type=int, choices=sorted(PREFILL_NAMES),
                    help="time the prompt (multi-query) step of this workload instead of the decode step")
    ap.add_argument("--prefill-cache", choices=["e4m3", "i8"], default="",
                    help="with --prefill: hold the pools in this 8-bit format (per-pool scales)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain block copy of known size (for HBM byte-counter scaling)")
    a = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}, WORLD_SIZE {world}): this decode path "
              "has no multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        return 2

    if a.calibrate_copy:
        print(json.dumps(calibrate_copy()), flush=True)
        return 0
    if a.prefill:
        return prefill_main(a)
    if a.swap:
        return swap_main(a)
    if a.head_scales:
        decode_config(a.config, True)                # refuses the 16-bit workloads
    cpu = None if a.no_cpu_baseline else cpu_baseline(a.config, a.cpu_sample_seqs, a.cpu_seconds, a.head_scales)
    if a.group_size > 1 and (a.graph or a.head_scales):
        raise SystemExit("--group-size is measured on its own (not with --graph or --head-scales)")
    case, wall, instrumented_wall, decode_ms, part_ms, kernel_ms, unfused_wall, cold, graphs, stream, parts = gpu_bench(
        a.config, a.steps, a.warmup, a.cold_iters, a.graph, a.head_scales, a.group_size)

    import paged_kv_cache_423_amd as pkv
    merged = pkv.decode_workspace_bytes(case.S, case.H, case.D, case.BS, case.MB) > 0
    kvb = case.kv_bytes
    eager_ms_step = wall / a.steps * 1e3
    ms_step = graphs["graph_appending_decode_ms"] if a.graph else eager_ms_step
    dec_avg = statistics.fmean(decode_ms)
    part_avg = statistics.fmean(part_ms)
    # with shared prefixes the roofline counts each physical row once: the
    # logical rate may exceed the peak through cache reuse, the unique one not
    uniq = case.unique_kv_bytes
    roof_bytes = min(uniq, kvb)
    # the partition kernel's own duration, from back-to-back launches queued
    # behind GPU work (in-step events of a host-bound step time enqueue gaps)
    achieved = roof_bytes / (kernel_ms / 1e3) / 1e9
    q = np.percentile(decode_ms, [10, 50, 90])
    cold_med = statistics.median(cold) if cold else None
    line = {
        "metric": "paged-attn decode K/V-read GB/s (% of HBM peak) and seq-heads/sec",
        "value": round(kvb / (ms_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"e4m3": "fp8-e4m3 KV / f16", "i8": "int8 KV / f16"}.get(case.cache_dtype, case.cache_dtype),
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[a.config] + (", one scale per head" if a.head_scales else "")
                        + (f", decoded in groups of {a.group_size}" if a.group_size > 1 else ""),
            "num_seqs": case.S, "num_heads": case.H, "head_size": case.D, "block_size": case.BS,
            "num_blocks": case.NB, "max_blocks_per_seq": case.MB,
            "context_tokens": int(case.context_lens.sum()),
            "kv_bytes_per_step": kvb,
            **({"unique_kv_bytes_per_step": uniq} if uniq < kvb else {}),
        },
        "pct_hbm_peak": round(100 * kvb / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 2),
        "seq_heads_per_s": round(case.S * case.H / (ms_step / 1e3), 1),
        "decode_ms": {"mean": round(dec_avg, 4), "p10": round(float(q[0]), 4), "p50": round(float(q[1]), 4),
                      "p90": round(float(q[2]), 4)},
        # the partition kernel: back to back on the device (the roofline's
        # duration), and between the in-step events (includes any host gap)
        "partition_kernel_ms": round(kernel_ms, 5),
        "partition_phase_in_step_ms_mean": round(part_avg, 4),
        # decode minus partition phase: the merge kernel, or only event overhead
        # when every context fits one partition and no merge is launched
        "merge_phase_ms_mean": round(dec_avg - part_avg, 4),
        "merge_kernel_launched": merged,
        "decode_cold_ms_median": None if cold_med is None else round(cold_med, 4),
        "decode_cold_GBps": None if cold_med is None else round(kvb / (cold_med / 1e3) / 1e9, 1),
        "step_mode": "hip-graph replay of the step, cache write fused into the decode, no timing events "
                     "(graph_comparison: the other forms in the same run)" if a.graph
                     else "eager calls (prepared once before the loop), "
                          + ("cache write as its own kernel before the decode (8-bit pools)"
                             if case.cache_dtype in ("e4m3", "i8") else "cache write fused into the "
                             + ("grouped decode" if a.group_size > 1 else "decode"))
                          + ", no timing events in the timed loop (decode_ms: a second pass of the same steps with "
                          f"events on every {EVENT_STRIDE}th step)",
        "eager_ms_per_step": round(eager_ms_step, 4),
        "instrumented_ms_per_step": round(instrumented_wall / a.steps * 1e3, 4),
        **({"graph_comparison": graphs} if graphs else {}),
        "unfused_ms_per_step": round(unfused_wall / a.steps * 1e3, 4),
        "components": component_report(case, parts),
        "pool": pool_report(case),
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_decode_group_kernel (the grouped decode's partition phase, writing the step's "
                       "tokens)" if a.group_size > 1
                       else "paged_decode_kernel (the decode's partition phase; its cache write runs as "
                       "reshape_and_cache_kernel first)" if case.cache_dtype in ("e4m3", "i8")
                       else "paged_decode_kernel (the decode's partition phase, writing the step's tokens)"),
            "duration": f"{COMPONENT_REPS} back-to-back launches queued behind GPU work, median of "
                        f"{COMPONENT_ROUNDS} rounds",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if a.head_scales else traffic_bytes(a.config, a.group_size),
            "bytes": "unique K/V rows (shared prefix once)" if uniq < kvb else "K/V rows read",
            "frac_of_stream_read": round(achieved / stream["GBps"], 4),
        },
        "stream_read": stream,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""GPU: pools larger than 4 GiB, with the mapped blocks spread across them.

A device with 288 GB of HBM holds per-layer pools of several GiB, where a
block's byte offset no longer fits 32 bits.  Each case here builds pools of
about 6.5 GB each for K and V (200,000 blocks of 32 KiB, or 400,000 of 16 KiB)
and places the step's blocks at random over the whole pool, so that about a
third of them lie past the 4 GiB mark:

* decode over bf16, E4M3 and INT8 pools (cache write, partition kernel, one
  sequence long enough for several partitions and the merge), against the
  oracle on every sequence, and the appending decode bit for bit against
  the separate calls;
* the device-side check of the step's index inputs (mask 0, as the oracle's
  validator finds) and the block gather of every sequence, bit for bit;
* the shared-prefix step with copy-on-write copies between blocks on both
  sides of the mark, as the per-sequence decode and bit for bit as the
  grouped appending decode, then a swap of blocks from both sides out to
  pinned host memory and back into free blocks past the mark;
* prompt attention over f16 and E4M3 pools, against the oracle.

The oracle runs on a compact pool holding the mapped blocks, renumbered (the
result depends only on the rows a table maps).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import checks as C
from gpu_common import check_step, oracle_step, require_gpu, run_gpu_step
from test_gpu_prefill import check as prefill_check
from test_gpu_prefill import oracle_run as prefill_oracle
from test_gpu_prefill import run_gpu as prefill_gpu

pytestmark = pytest.mark.gpu

TARGET_BYTES = 6.5e9                       # per pool
FOUR_GIB = 1 << 32


@pytest.fixture(autouse=True)
def _release_pools():
    yield
    torch.cuda.empty_cache()                # several GiB per case: give them back between cases


def _block_bytes(H, BS, D, dtype):
    return H * BS * D * {"bf16": 2, "f16": 2, "e4m3": 1, "i8": 1}[dtype]


def _past_mark(ids, block_bytes):
    ids = np.asarray(ids, dtype=np.int64).ravel()
    return int(np.count_nonzero(ids * block_bytes >= FOUR_GIB))


DECODE = {
    "bf16": replace(W.CONFIGS[3], name="large-pool-bf16", S=24, H=8, MB=320),
    "e4m3": replace(W.CONFIGS[5], name="large-pool-e4m3", S=24, H=8, MB=160),
    "i8": replace(W.CONFIGS[6], name="large-pool-i8", S=24, H=8, MB=160),
}


@pytest.mark.parametrize("fmt", sorted(DECODE))
def test_decode_over_pools_past_four_gib(fmt):
    pkv = require_gpu()
    cfg = DECODE[fmt]
    rng = np.random.Generator(np.random.PCG64(4096))
    lens = np.concatenate([rng.integers(200, 1501, cfg.S - 1), [5000]]).astype(np.int64)
    blocks = int(sum(-(-int(n) // cfg.BS) for n in lens))
    bb = _block_bytes(cfg.H, cfg.BS, cfg.D, cfg.cache_dtype)
    case = W.make_case(cfg, device="cuda", context_lens=lens, NB_slack=TARGET_BYTES / bb / blocks)
    used = np.concatenate([case.block_tables[s, :-(-int(case.context_lens[s]) // cfg.BS)] for s in range(case.S)])
    print(f"large pool {fmt}: NB={case.NB} ({case.NB * bb / 2**30:.2f} GiB per pool), "
          f"{_past_mark(used, bb)} of {used.size} mapped blocks and "
          f"{_past_mark(case.slot_mapping // cfg.BS, bb)} of {case.S} written slots past 4 GiB", flush=True)
    assert case.NB * bb > FOUR_GIB + (1 << 30)
    assert _past_mark(used, bb) > used.size // 5 and _past_mark(case.slot_mapping // cfg.BS, bb) > 0
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    err = check_step(case, g, o, f"large pool {fmt}")
    print(f"large pool {fmt}: max abs error {err:.3g}", flush=True)

    # the appending decode from the pre-step pools equals the two calls bit for bit
    out = torch.empty_like(g.out)
    pkv.paged_attention_decode_append(out, case.q, case.key, case.value, g.k_pre, g.v_pre,
                                      torch.from_numpy(case.slot_mapping).to("cuda"), g.block_tables,
                                      g.context_lens, case.scale, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), g.out.view(torch.uint8)), f"{fmt}: appending decode output differs"
    idx = torch.from_numpy(o.blocks[o.mapped]).to("cuda")
    for a, b, n in ((g.k_pre, g.k_post, "K"), (g.v_pre, g.v_post, "V")):
        assert torch.equal(a.index_select(0, idx).view(torch.uint8), b.index_select(0, idx).view(torch.uint8)), \
            f"{fmt}: appending decode {n} pool differs"

    slots = torch.from_numpy(case.slot_mapping).to("cuda")
    want = C.step_input_violations(case.block_tables, case.context_lens, cfg.BS, case.NB, case.slot_mapping,
                                   None, append=True)
    assert pkv.check_step_inputs(g.block_tables, g.context_lens, cfg.BS, case.NB, slots, None, True) == want == 0

    # the block gather of every sequence from the updated pools
    remap = {int(b): i for i, b in enumerate(o.blocks)}
    mini = np.zeros_like(case.block_tables)
    for s in range(case.S):
        nb = -(-int(case.context_lens[s]) // cfg.BS)
        mini[s, :nb] = [remap[int(b)] for b in case.block_tables[s, :nb]]
    wk, wv, cu = oracle.gather_kv(o.k_post, o.v_post, mini, case.context_lens)
    gk = torch.empty((int(cu[-1]), cfg.H, cfg.D), dtype=g.k_post.dtype, device="cuda")
    gv = torch.empty_like(gk)
    pkv.gather_kv(gk, gv, torch.from_numpy(cu.astype(np.int32)).to("cuda"), g.k_post, g.v_post, g.block_tables,
                  g.context_lens)
    torch.cuda.synchronize()
    assert np.array_equal(W.bits(gk, cfg.cache_dtype), wk) and np.array_equal(W.bits(gv, cfg.cache_dtype), wv), \
        f"{fmt}: gathered rows differ"


def test_copy_on_write_step_over_a_pool_past_four_gib():
    pkv = require_gpu()
    cfg = replace(W.CONFIGS[4], name="large-pool-cow-f16", H=8)
    # the same seed draws the same lengths at one head: its pool size gives
    # the blocks the step needs, NB = ceil(1.25 * need) + copies + 1
    probe = W.make_case(replace(cfg, H=1), device="cpu")
    need = (probe.NB - 1 - probe.copy_pairs.shape[0]) / 1.25
    bb = _block_bytes(cfg.H, cfg.BS, cfg.D, cfg.cache_dtype)
    case = W.make_case(cfg, device="cuda", NB_slack=TARGET_BYTES / bb / need)
    pairs = case.copy_pairs
    print(f"large pool copy-on-write: NB={case.NB}, {pairs.shape[0]} copies, "
          f"{_past_mark(pairs[:, 0], bb)} sources and {_past_mark(pairs[:, 1], bb)} destinations past 4 GiB",
          flush=True)
    assert case.NB * bb > FOUR_GIB + (1 << 30)
    assert _past_mark(pairs, bb) > 0 and _past_mark(pairs, bb) < pairs.size
    g = run_gpu_step(pkv, case)
    o = oracle_step(case, g.k_pre, g.v_pre)
    err = check_step(case, g, o, "large pool copy-on-write")
    print(f"large pool copy-on-write: max abs error {err:.3g}", flush=True)

    # the same step as the grouped appending decode (groups of 8: shared
    # blocks read once per chunk, the new tokens stored by the kernel), from
    # the pools before the step: output and both whole pools bit for bit
    kc, vc = g.k_pre.clone(), g.v_pre.clone()
    pkv.copy_blocks(kc, vc, torch.from_numpy(pairs).to("cuda"))
    out = torch.empty_like(case.q)
    slots = torch.from_numpy(case.slot_mapping).to("cuda")
    ws = pkv.alloc_decode_workspace(case.S, case.H, case.D, case.BS, case.MB)
    pkv.paged_attention_decode_grouped(out, case.q, kc, vc, g.block_tables, g.context_lens, case.scale, 8,
                                       key=case.key, value=case.value, slot_mapping=slots, workspace=ws)
    torch.cuda.synchronize()
    for name, x, y in (("output", out, g.out), ("K pool", kc, g.k_post), ("V pool", vc, g.v_post)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"large pool grouped decode: {name} differs"
    del kc, vc
    print("large pool grouped appending decode: bitwise the per-sequence step", flush=True)

    # swap: the blocks of the first two groups out to pinned host memory, then
    # back into blocks no sequence maps, past the mark; each destination
    # block is then a copy of its source block, bit for bit
    mapped = np.zeros(case.NB, dtype=bool)
    for s in range(16):
        mapped[case.block_tables[s, :-(-int(case.context_lens[s]) // cfg.BS)]] = True
    out_ids = np.nonzero(mapped)[0]
    assert _past_mark(out_ids, bb) > 0 and _past_mark(out_ids, bb) < out_ids.size
    high_free = np.nonzero(~mapped)[0]
    high_free = high_free[high_free * bb >= FOUR_GIB + (1 << 30)]
    in_ids = np.random.Generator(np.random.PCG64(4098)).choice(high_free, out_ids.size, replace=False)
    n = out_ids.size
    hk = torch.zeros((n,) + tuple(g.k_post.shape[1:]), dtype=g.k_post.dtype, pin_memory=True)
    hv = torch.zeros((n,) + tuple(g.v_post.shape[1:]), dtype=g.v_post.dtype, pin_memory=True)
    out_pairs = torch.from_numpy(np.stack([out_ids, np.arange(n)], 1).astype(np.int32)).to("cuda")
    in_pairs = torch.from_numpy(np.stack([np.arange(n), in_ids], 1).astype(np.int32)).to("cuda")
    pkv.swap_blocks(hk, hv, g.k_post, g.v_post, out_pairs)
    torch.cuda.synchronize()
    pkv.swap_blocks(g.k_post, g.v_post, hk, hv, in_pairs)
    torch.cuda.synchronize()
    src = torch.from_numpy(out_ids).to("cuda")
    dst = torch.from_numpy(in_ids.astype(np.int64)).to("cuda")
    for pool, host, name in ((g.k_post, hk, "K"), (g.v_post, hv, "V")):
        assert torch.equal(host.view(torch.uint8), pool.index_select(0, src).cpu().view(torch.uint8)), \
            f"swap out: {name} host blocks differ"
        assert torch.equal(pool.index_select(0, dst).view(torch.uint8), pool.index_select(0, src).view(torch.uint8)), \
            f"swap in: {name} blocks differ"
    print(f"large pool swap: {n} blocks out ({_past_mark(out_ids, bb)} past 4 GiB) and back in past 5 GiB",
          flush=True)


@pytest.mark.parametrize("cache", ["", "e4m3"], ids=["f16-pools", "e4m3-pools"])
def test_prefill_over_pools_past_four_gib(cache):
    pkv = require_gpu()
    cfg = replace(W.PREFILL_CONFIGS[2], name="large-pool-prompts", S=8, H=8, cache_dtype=cache)
    rng = np.random.Generator(np.random.PCG64(4097))
    cached = rng.integers(100, 700, cfg.S)
    new = rng.integers(40, 300, cfg.S)
    need = int(sum(-(-int(c + n) // cfg.BS) for c, n in zip(cached, new)))
    bb = _block_bytes(cfg.H, cfg.BS, cfg.D, cfg.pool_dtype)
    case = W.make_prefill_case(cfg, device="cuda", q_lens=new, cached=cached, NB_slack=TARGET_BYTES / bb / need)
    used = np.concatenate([case.block_tables[s, :-(-int(case.context_lens[s]) // cfg.BS)] for s in range(case.S)])
    print(f"large pool prompts {cfg.pool_dtype}: NB={case.NB}, {_past_mark(used, bb)} of {used.size} mapped "
          f"blocks past 4 GiB", flush=True)
    assert case.NB * bb > FOUR_GIB + (1 << 30)
    assert _past_mark(used, bb) > used.size // 5
    k_pre, v_pre, gk, gv, gout = prefill_gpu(pkv, case)
    o = prefill_oracle(case, k_pre, v_pre)
    err = prefill_check(case, gk, gv, gout, o, f"large pool prompts {cfg.pool_dtype}")
    print(f"large pool prompts {cfg.pool_dtype}: max abs error {err:.3g}", flush=True)

"""Host block bookkeeping and the seeded workloads (CPU).

The block manager reproduces the pages' worked examples (the append
walk-through of "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战" §2.1 and the
slot-mapping example of the l189.com article §2.2), its copy-on-write
follows the same page's §2.2, and the generated workloads have the shapes,
lengths, sharing and poison padding their descriptions ask for.
"""

import json
import os

import numpy as np
import pytest

import workloads as W
import workloads.configs as WC
from workloads.blocks import BlockManager, BlockPool, OutOfBlocks


def test_append_walkthrough(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "append_walkthrough.json")))
    bm = BlockManager(g["block_size"], BlockPool(len(g["free_order"]), g["free_order"]))
    bm.add_sequence(0, g["prompt_tokens"])
    assert bm.table(0) == g["steps"][0]["table_after"]
    for step in g["steps"][1:]:
        slot, copy = bm.append_slot(0)
        assert copy is None
        assert slot == step["slot"] and bm.table(0) == step["table_after"]


def test_slot_mapping_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "slot_mapping_example.json")))
    BS = g["block_size"]
    # free pool order that hands A block 5, then B block 3, then A block 8
    order = [5, 3, 8] + [b for b in range(10) if b not in (5, 3, 8)]
    bm = BlockManager(BS, BlockPool(10, order))
    bm.add_sequence("A", 16)
    bm.add_sequence("B", 16)
    for _ in range(16):
        bm.append_slot("A")
    assert bm.table("A") == g["tables"]["A"] and bm.table("B") == g["tables"]["B"]
    for e in g["expect_slots"]:
        assert bm.slot_of(e["seq"], e["token"]) == e["slot"]


def test_copy_on_write_and_refcounts():
    bm = BlockManager(4, BlockPool(8))
    bm.add_sequence(0, 6)                 # blocks 0, 1 (block 1 half full)
    bm.fork(0, 1)
    assert bm.pool.refcount == {0: 2, 1: 2}
    slot, copy = bm.append_slot(1)        # writes into shared block 1 -> copy first
    assert copy == (1, 2) and bm.table(1) == [0, 2] and slot == 2 * 4 + 2
    assert bm.pool.refcount == {0: 2, 1: 1, 2: 1}
    slot, copy = bm.append_slot(0)        # block 1 is now private to seq 0
    assert copy is None and slot == 1 * 4 + 2
    assert bm.make_private(0, 0) == (0, 3) and bm.make_private(1, 0) is None
    bm.free_sequence(0)
    bm.free_sequence(1)
    assert bm.pool.refcount == {} and bm.pool.num_free == 8


def test_pool_exhaustion():
    bm = BlockManager(16, BlockPool(2))
    bm.add_sequence(0, 32)
    with pytest.raises(OutOfBlocks):
        bm.append_slot(0)
    with pytest.raises(ValueError):
        BlockPool(3, [0, 1, 1])


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_workload_shapes_and_padding(idx):
    cfg = W.CONFIGS[idx]
    S = cfg.S if idx in (1, 2) else 16
    c = W.make_case(cfg, S=S, H=2)
    assert c.k_cache.shape == (c.NB, 2, cfg.BS, cfg.D) and c.q.shape == (c.S, 2, cfg.D)
    assert c.block_tables.shape == (c.S, c.MB) and c.block_tables.dtype == np.int32
    n = c.context_lens
    if cfg.ctx_dist != "shared":
        assert n.min() >= cfg.ctx_lo and n.max() <= cfg.ctx_hi
    if idx in (1, 2):
        assert c.NB == cfg.NB_fixed
    # each new token's slot sits in the block the table maps for position n-1
    for s in range(c.S):
        blk = c.block_tables[s, (n[s] - 1) // c.BS]
        assert c.slot_mapping[s] == blk * c.BS + (n[s] - 1) % c.BS
        nb = -(-int(n[s]) // c.BS)
        assert (c.block_tables[s, nb:] == c.poison_block).all()
    # distinct slots; the poison block is never mapped
    assert np.unique(c.slot_mapping).size == c.S
    for s in range(c.S):
        nb = -(-int(n[s]) // c.BS)
        assert c.poison_block not in c.block_tables[s, :nb]
    # the poison block and every new token's slot are NaN before the write
    kc = c.k_cache
    if cfg.cache_dtype == "e4m3":
        assert (kc[c.poison_block] == 0x7F).all()
    elif cfg.cache_dtype == "i8":
        assert (kc[c.poison_block] == -128).all()
        for s in range(c.S):
            b, o = divmod(int(c.slot_mapping[s]), c.BS)
            assert (kc[b, :, o] == -128).all()
    else:
        assert kc[c.poison_block].float().isnan().all()
        for s in range(c.S):
            b, o = divmod(int(c.slot_mapping[s]), c.BS)
            assert kc[b, :, o].float().isnan().all()


def test_shared_prefix_workload():
    c = W.make_case(W.CONFIGS[4], S=64, H=1)
    assert c.S == 64 and len(c.groups) == 8
    assert c.copy_pairs.shape == (56, 2)
    # before the step each group maps one prefix; after it, writers 0..6 own a copy of block 31
    for grp in c.groups:
        pre = [c.pre_tables[s][:32] for s in grp]
        assert all(p == pre[0] for p in pre)
        post31 = [int(c.block_tables[s, 31]) for s in grp]
        assert post31[-1] == pre[0][31] and len(set(post31)) == 8
        for s in grp:
            assert list(c.block_tables[s, :31]) == pre[0][:31]
    src = set(c.copy_pairs[:, 0].tolist())
    assert len(src) == 8
    assert c.unique_kv_bytes < c.kv_bytes


def test_shared_prefix_on_write_workload():
    c = W.make_case(W.CONFIG_4_ON_WRITE, S=16, H=1)
    assert (c.context_lens == 501).all()
    assert c.copy_pairs.shape == (14, 2)
    for grp in c.groups:
        offs = c.slot_mapping[grp] % 16
        assert (offs == 500 % 16).all()
        blocks = c.slot_mapping[grp] // 16
        assert len(set(blocks.tolist())) == len(grp)     # every writer ends in its own block


def test_seeded_determinism():
    a = W.make_case(W.CONFIGS[5], S=8, H=1)
    b = W.make_case(W.CONFIGS[5], S=8, H=1)
    assert (a.context_lens == b.context_lens).all() and (a.block_tables == b.block_tables).all()
    assert a.k_scale == b.k_scale and 0.01 <= a.k_scale <= 0.1
    assert (a.k_cache == b.k_cache).all()


def test_loguniform_lengths():
    rng = np.random.default_rng(0)
    n = W.draw_context_lens(W.CONFIGS[5], rng, 200_000)
    assert n.min() >= 128 and n.max() == 4096
    # mean of min(4096, floor(exp(U[ln 128, ln 4097)))) is about 1145
    assert abs(n.mean() - 1145) < 15


def test_prefill_8bit_pools_keep_the_16bit_draws():
    """An 8-bit pool format changes only the pools and the two scales: the
    lengths, placement, slots and q / key / value match the 16-bit case of
    the same seed, the scales lie in the configured range, and unmapped
    blocks hold the poison byte."""
    from dataclasses import replace
    base = W.PREFILL_CONFIGS[1]
    c16 = W.make_prefill_case(base)
    for fmt, torch_dtype, poison in (("e4m3", "uint8", WC.E4M3_NAN_BYTE), ("i8", "int8", WC.I8_POISON)):
        c8 = W.make_prefill_case(replace(base, cache_dtype=fmt))
        assert c8.pool_dtype == fmt and str(c8.k_cache.dtype).endswith(torch_dtype)
        for name in ("context_lens", "q_lens", "cu_q_lens", "block_tables", "slot_mapping", "copy_pairs"):
            assert np.array_equal(getattr(c8, name), getattr(c16, name)), name
        for name in ("q", "key", "value"):
            assert bool((getattr(c8, name) == getattr(c16, name)).all()), name
        for sc in (c8.k_scale, c8.v_scale):
            assert base.scale_lo <= sc <= base.scale_hi
        assert int(c8.k_cache[c8.poison_block].flatten()[0]) == poison
    assert c16.pool_dtype == base.dtype and (c16.k_scale, c16.v_scale) == (1.0, 1.0)


def test_head_scale_workloads_keep_the_per_pool_draws():
    """One scale per head changes only the scales and the stored bytes: the
    lengths, placement, slots and q / key / value match the per-pool
    workload of the same seed; each head's scales lie in the configured
    range and differ; each head's bytes are that head's values over its own
    scale."""
    import oracle
    for per_pool, per_head in ((W.CONFIGS[5], W.CONFIG_5_HEAD_SCALES), (W.CONFIGS[6], W.CONFIG_6_HEAD_SCALES)):
        a = W.make_case(per_pool, S=16, H=4)
        b = W.make_case(per_head, S=16, H=4)
        for name in ("context_lens", "block_tables", "slot_mapping", "copy_pairs"):
            assert np.array_equal(getattr(a, name), getattr(b, name)), name
        for name in ("q", "key", "value"):
            assert bool((getattr(a, name) == getattr(b, name)).all()), name
        for sc in (b.k_scale, b.v_scale):
            assert sc.shape == (4,) and sc.dtype == np.float32 and np.unique(sc).size == 4
            assert ((sc >= per_head.scale_lo) & (sc <= per_head.scale_hi)).all()
        # the same N(0, 1) draws, quantised over two different scales: the values agree within
        # two rounding steps of the coarser one (E4M3: 2^-3 relative; INT8: one scale)
        blk = int(b.block_tables[0, 0])
        for h in range(4):
            xa = W.bits(a.k_cache[blk, h], per_pool.cache_dtype)
            xb = W.bits(b.k_cache[blk, h], per_head.cache_dtype)
            va = oracle.decode(xa, per_pool.cache_dtype) * a.k_scale
            vb = oracle.decode(xb, per_head.cache_dtype) * float(b.k_scale[h])
            ok = np.isfinite(va) & np.isfinite(vb)
            assert np.allclose(va[ok], vb[ok], rtol=0.13, atol=2 * max(a.k_scale, float(b.k_scale[h])))
    c = W.make_prefill_case(__import__("dataclasses").replace(W.PREFILL_CONFIGS[1], cache_dtype="i8",
                                                                head_scales=True))
    assert c.k_scale.shape == (c.H,) and c.v_scale.shape == (c.H,)

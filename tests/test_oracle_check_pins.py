"""Pins of the oracle's step-input validation (oracle.checks), CPU only.

The validator states, one condition per bit, when a step's block tables,
context lengths, slot mapping and copy pairs are well formed.  It is pinned
by things other than itself:

* every generated workload step (all decode workloads, the copy-on-write
  variant, the prompt workloads) is well formed by construction: mask 0;
* a single planted fault sets exactly its own bit;
* the copy-on-write rule ("在A10G上榨干LLaMA-7B" §2.2): on the shared-prefix
  workload whose append lands inside the shared block, the tables *before*
  the copy make the write land in a block eight sequences map (bit 7), the
  tables after it do not;
* on random small steps, the range and collision bits agree with where the
  oracle's own operations refuse their inputs (reshape_and_cache,
  copy_blocks, paged_attention_decode), and the appending and shared-write
  bits agree with the effect of the writes, found by brute force: writing
  distinct markers and gathering every sequence's rows back.
"""

from __future__ import annotations

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
import workloads as W
from oracle import checks as C

BITS = [C.CONTEXT_LEN, C.BLOCK_ID, C.SLOT_RANGE, C.SLOT_DUP, C.PAIR_RANGE, C.PAIR_OVERLAP, C.APPEND_SLOT,
        C.SHARED_WRITE]


def test_bits_are_distinct_single_bits():
    assert len(set(BITS)) == 8 and all(b & (b - 1) == 0 for b in BITS) and sum(BITS) == 0xFF


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_generated_decode_steps_are_well_formed(idx):
    case = W.make_case(W.CONFIGS[idx], device="cpu", S=min(W.CONFIGS[idx].S, 64), H=1)
    m = C.step_input_violations(case.block_tables, case.context_lens, case.BS, case.NB, case.slot_mapping,
                                case.copy_pairs, append=True)
    assert m == 0, hex(m)


def test_copy_on_write_variant_is_well_formed_after_the_copy_and_not_before():
    case = W.make_case(W.CONFIG_4_ON_WRITE, device="cpu", H=1)
    assert len(case.copy_pairs) > 0
    after = C.step_input_violations(case.block_tables, case.context_lens, case.BS, case.NB, case.slot_mapping,
                                    case.copy_pairs, append=True)
    assert after == 0, hex(after)
    pre = np.full_like(case.block_tables, case.poison_block)
    for s, row in enumerate(case.pre_tables):
        pre[s, :len(row)] = row
    # before the copy the writers' last logical block is still the shared one;
    # give the pre-step tables the step's lengths (the write goes into the
    # block holding position n - 1, which the shared block is)
    n_pre = case.context_lens
    before = C.step_input_violations(pre, n_pre, case.BS, case.NB, case.slot_mapping, None, append=False)
    assert before & C.SHARED_WRITE, hex(before)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_generated_prompt_steps_are_well_formed(idx):
    cfg = W.PREFILL_CONFIGS[idx]
    case = W.make_prefill_case(cfg, device="cpu", H=1, S=min(cfg.S, 16))
    m = C.step_input_violations(case.block_tables, case.context_lens, case.BS, case.NB, case.slot_mapping,
                                case.copy_pairs)
    assert m == 0, hex(m)


def _small_step():
    """A well-formed appending step by hand: 3 sequences, BS 4, NB 12."""
    BS, NB = 4, 12
    tables = np.array([[3, 7, 0], [5, 0, 0], [9, 2, 11]], dtype=np.int32)
    lens = np.array([6, 4, 9], dtype=np.int32)
    # slot of position n - 1 of each sequence
    slots = np.array([7 * BS + 1, 5 * BS + 3, 11 * BS + 0], dtype=np.int32)
    pairs = np.array([[1, 4], [6, 8]], dtype=np.int32)
    return tables, lens, slots, pairs, BS, NB


def test_hand_step_is_well_formed():
    t, n, s, p, BS, NB = _small_step()
    assert C.step_input_violations(t, n, BS, NB, s, p, append=True) == 0


@pytest.mark.parametrize("fault,bit", [
    ("len_over", C.CONTEXT_LEN), ("len_negative", C.CONTEXT_LEN), ("block_past", C.BLOCK_ID),
    ("block_negative", C.BLOCK_ID), ("slot_past", C.SLOT_RANGE), ("slot_dup", C.SLOT_DUP),
    ("pair_past", C.PAIR_RANGE), ("pair_dst_repeat", C.PAIR_OVERLAP), ("pair_dst_is_src", C.PAIR_OVERLAP),
    ("append_wrong_offset", C.APPEND_SLOT), ("append_zero_len", C.APPEND_SLOT),
    ("shared_write", C.SHARED_WRITE), ("unused_entry_is_ignored", 0), ("padding_slot_is_allowed", 0),
])
def test_a_single_fault_sets_its_own_bit(fault, bit):
    t, n, s, p, BS, NB = _small_step()
    append = True
    if fault == "len_over":
        n[1] = 3 * BS + 1                      # past MB * BS = 12 (entries clamp to the row: all in range)
        s[1] = -1                              # so the append contract does not speak too
    elif fault == "len_negative":
        n[1] = -2
        s[1] = -1
    elif fault == "block_past":
        t[0, 0] = NB
    elif fault == "block_negative":
        t[2, 1] = -1
    elif fault == "slot_past":
        s[0] = NB * BS
        append = False
    elif fault == "slot_dup":
        s[2] = s[0]
        append = False
    elif fault == "pair_past":
        p[1, 0] = NB
    elif fault == "pair_dst_repeat":
        p[1, 1] = p[0, 1]
    elif fault == "pair_dst_is_src":
        p[1, 1] = p[0, 0]
    elif fault == "append_wrong_offset":
        s[0] += 1
    elif fault == "append_zero_len":
        n[1] = 0
    elif fault == "shared_write":
        t[1, 0] = 7                            # sequence 1 now maps sequence 0's last block too
        s[1] = -1                              # (its own write skipped: only the shared write remains)
    elif fault == "unused_entry_is_ignored":
        t[1, 1] = NB + 5                       # logical block 1 of a 4-token sequence is never read
    elif fault == "padding_slot_is_allowed":
        s[2] = -7
    got = C.step_input_violations(t, n, BS, NB, s, p, append=append)
    assert got == bit, (fault, hex(got))


# ---------------------------------------------------------------- random steps

def _random_step(seed: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    S, MB = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    BS = int(rng.choice([1, 2, 4]))
    NB = int(rng.integers(2, 10))
    bad = rng.random() < 0.5                   # about half the steps carry faults
    lens = rng.integers(0 if not bad else -1, MB * BS + (2 if bad else 1), S)
    tables = rng.integers(-1 if bad else 0, NB + (1 if bad else 0), (S, MB))
    slots = np.empty(S, dtype=np.int64)
    for i in range(S):                         # mostly the appending slot, sometimes anything
        n = min(max(int(lens[i]), 0), MB * BS)
        if n > 0 and rng.random() < 0.8:
            slots[i] = tables[i, (n - 1) // BS] * BS + (n - 1) % BS
        else:
            slots[i] = rng.integers(-1, NB * BS + (1 if bad else 0))
    npairs = int(rng.integers(0, 4))
    pairs = rng.integers(0 if not bad else -1, NB + (1 if bad else 0), (npairs, 2))
    return (tables.astype(np.int32), lens.astype(np.int32), slots.astype(np.int32),
            pairs.astype(np.int32), BS, NB)


def _raises(fn) -> bool:
    try:
        fn()
    except (ValueError, IndexError):
        return True
    return False


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_range_and_collision_bits_agree_with_the_operations(seed):
    t, n, s, p, BS, NB = _random_step(seed)
    m = C.step_input_violations(t, n, BS, NB, s, p)
    S, H, D = len(n), 1, 2
    pool = np.zeros((NB, H, BS, D), dtype=np.uint32)
    key = np.zeros((S, H, D), dtype=np.uint32)
    write_refused = _raises(lambda: oracle.reshape_and_cache(key, key, pool, pool, s, "f32", "f32"))
    assert write_refused == bool(m & (C.SLOT_RANGE | C.SLOT_DUP)), hex(m)
    copy_refused = _raises(lambda: oracle.copy_blocks(pool, pool, p))
    assert copy_refused == bool(m & (C.PAIR_RANGE | C.PAIR_OVERLAP)), hex(m)
    q = np.zeros((S, H, D), dtype=np.uint32)
    decode_refused = _raises(lambda: oracle.paged_attention_decode(q, pool, pool, t, n, 1.0, "f32", "f32"))
    assert decode_refused == bool(m & (C.CONTEXT_LEN | C.BLOCK_ID)), hex(m)


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_append_and_shared_write_bits_agree_with_the_writes(seed):
    t, n, s, p, BS, NB = _random_step(seed)
    m = C.step_input_violations(t, n, BS, NB, s, None, append=True)
    if m & (C.CONTEXT_LEN | C.BLOCK_ID | C.SLOT_RANGE | C.SLOT_DUP):
        return                                 # the writes or gathers are undefined: nothing to compare
    S, MB = t.shape
    # pool values 1 .. NB*BS by slot, new tokens' markers far above them
    pool = (np.arange(NB * BS, dtype=np.uint32) + 1).reshape(NB, 1, BS, 1)
    key = (np.arange(S, dtype=np.uint32) + 10_000).reshape(S, 1, 1)
    after, _ = oracle.reshape_and_cache(key, key, pool, pool, s, "f32", "f32")

    # appending contract: every sequence with a slot reads its own new token
    # at position n - 1, and n > 0
    ok = True
    for i in range(S):
        if s[i] < 0:
            continue
        if n[i] == 0:
            ok = False
            continue
        rows = oracle.gather_kv(after, after, t[i:i + 1], n[i:i + 1])[0]
        ok &= int(rows[n[i] - 1, 0, 0]) == 10_000 + i
    assert ok == (not (m & C.APPEND_SLOT)), hex(m)

    # shared write: some written slot changes more than one used logical
    # block (whole blocks gathered, so offsets past a sequence's length count)
    nblk = -(-np.maximum(n, 0) // BS)
    before_rows = [oracle.gather_kv(pool, pool, t[i:i + 1], [int(nblk[i]) * BS])[0] for i in range(S)]
    after_rows = [oracle.gather_kv(after, after, t[i:i + 1], [int(nblk[i]) * BS])[0] for i in range(S)]
    shared = False
    for i in range(S):
        if s[i] < 0:
            continue
        touched = 0
        for j in range(S):
            for b in range(int(nblk[j])):
                blk_before = before_rows[j][b * BS:(b + 1) * BS]
                blk_after = after_rows[j][b * BS:(b + 1) * BS]
                if np.any(blk_after == 10_000 + i) and not np.any(blk_before == 10_000 + i):
                    touched += 1
        shared |= touched > 1
    assert shared == bool(m & C.SHARED_WRITE), hex(m)

"""The oracle's validation of one step's device-side index inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (titles as published):

* [P1] "vLLM-v0.17.1技术解析：PagedAttention内存管理与显存优化技巧"
* [P2] "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战"
* [P3] the l189.com article on KV cache, PagedAttention, slot mapping and
  CUDA graphs (www.l189.com/news/180929)

A step hands the device three index structures: the block tables with the
context lengths ([P1] §2.2, [P2] §2.1), the int32 slot mapping of the new
tokens ([P3] §2.2) and the copy-on-write block pairs ([P2] §2.2).  The
operations on them are defined only when the indices stay inside the pool and
do not collide; this module states those conditions one by one and reports
which of them a step breaks, as a bit mask:

=====  ==========================================================================
bit    condition broken
=====  ==========================================================================
0      a context length lies outside [0, MB * BS]
1      a used table entry (logical block j < ceil(n / BS), n clamped into
       [0, MB * BS]) names a block outside [0, NB)
2      a slot is at or past NB * BS (negative slots are padding, allowed)
3      two tokens name the same slot
4      a copy pair names a block outside [0, NB)
5      copy destinations repeat, or a destination is also a source
6      appending step only (one new token per sequence): a sequence's slot is
       not the slot of its position n - 1 through its table, or n = 0 with a
       slot given ([P2] §2.1: the generated token is stored in the sequence's
       last block, then used)
7      a written slot lies in a block that more than one used table entry
       maps ([P2] §2.2: a block is copied before a write while it is shared)
=====  ==========================================================================

Plain Python over sets and counters; nothing here is shared with the device
checks.
"""

from __future__ import annotations

from collections import Counter

import numpy as np

CONTEXT_LEN = 1 << 0
BLOCK_ID = 1 << 1
SLOT_RANGE = 1 << 2
SLOT_DUP = 1 << 3
PAIR_RANGE = 1 << 4
PAIR_OVERLAP = 1 << 5
APPEND_SLOT = 1 << 6
SHARED_WRITE = 1 << 7


def step_input_violations(block_tables, context_lens, BS: int, NB: int, slot_mapping=None, pairs=None,
                          append: bool = False) -> int:
    """Bit mask of the conditions (module docstring) that a step's index
    inputs break; 0 for a well-formed step.

    block_tables int [S, MB], context_lens int [S], slot_mapping int [T] or
    None, pairs int [N, 2] or None.  With append=True the slot mapping holds
    one slot per sequence (T == S) and bit 6 is checked as well.
    """
    tables = np.asarray(block_tables, dtype=np.int64)
    lens = [int(x) for x in np.asarray(context_lens, dtype=np.int64).reshape(-1)]
    S = len(lens)
    MB = tables.shape[1] if tables.ndim == 2 else 0
    if tables.shape[0] != S and S:
        raise ValueError("one table row per sequence")
    slots = [] if slot_mapping is None else [int(x) for x in np.asarray(slot_mapping, dtype=np.int64).reshape(-1)]
    prs = [] if pairs is None else [(int(a), int(b)) for a, b in np.asarray(pairs, dtype=np.int64).reshape(-1, 2)]
    if append and len(slots) != S:
        raise ValueError("an appending step has one slot per sequence")

    mask = 0
    maps = Counter()                 # block id -> used table entries naming it
    used_n = []                      # each sequence's length clamped into [0, MB * BS]
    for s in range(S):
        n = lens[s]
        if n < 0 or n > MB * BS:
            mask |= CONTEXT_LEN
        n = min(max(n, 0), MB * BS)
        used_n.append(n)
        for j in range(-(-n // BS)):
            b = int(tables[s, j])
            if b < 0 or b >= NB:
                mask |= BLOCK_ID
            else:
                maps[b] += 1

    seen = set()
    for slot in slots:
        if slot < 0:
            continue
        if slot >= NB * BS:
            mask |= SLOT_RANGE
            continue
        if slot in seen:
            mask |= SLOT_DUP
        seen.add(slot)
        if maps[slot // BS] > 1:
            mask |= SHARED_WRITE

    srcs, dsts = set(), []
    for src, dst in prs:
        if not (0 <= src < NB and 0 <= dst < NB):
            mask |= PAIR_RANGE
            continue
        srcs.add(src)
        dsts.append(dst)
    if len(set(dsts)) != len(dsts) or any(d in srcs for d in dsts):
        mask |= PAIR_OVERLAP

    if append:
        for s in range(S):
            slot, n = slots[s], used_n[s]
            if slot < 0:
                continue
            if n == 0:
                mask |= APPEND_SLOT
                continue
            t = n - 1
            b = int(tables[s, t // BS])
            if slot != b * BS + t % BS:
                mask |= APPEND_SLOT
    return mask

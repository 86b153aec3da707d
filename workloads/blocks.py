"""Host-side block bookkeeping that produces the decode step's index inputs.

This module makes inputs; it holds none of the kernels' arithmetic (no
attention, no number conversion).  It plays the part of the block manager the
pages sketch:

* a free pool of physical block ids, handed out one at a time
  ("vLLM-v0.17.1技术解析：PagedAttention内存管理与显存优化技巧" §2.2 keeps
  free blocks in a queue; "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战"
  §2.2 keeps a list; the l189.com article www.l189.com/news/180929 §2.3 gives
  the allocate / free interface);
* a per-sequence block table from logical to physical blocks;
* the append rule: a generated token goes into the sequence's last block
  while it has room, and a fresh block is mapped only once that block is
  full ("在A10G上榨干LLaMA-7B" §2.1, its three-step walk-through);
* sharing of whole blocks between sequences with a common prefix, with
  reference counts, and copy-on-write when a sequence is about to write a
  block that someone else still maps ("在A10G上榨干LLaMA-7B" §2.2).

Slots are numbered physical_block * block_size + offset (l189.com §2.2).
The free list is served first-in first-out from an order given by the caller;
a seeded permutation of all block ids gives the random physical placement the
workloads ask for.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    """The free pool is empty."""


class BlockPool:
    """Free list plus reference counts over physical ids 0 .. num_blocks-1."""

    def __init__(self, num_blocks: int, order: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        order = list(range(num_blocks)) if order is None else [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of all block ids")
        self.num_blocks = num_blocks
        self._free: List[int] = list(order)
        self._head = 0
        self.refcount: Dict[int, int] = {}

    @property
    def num_free(self) -> int:
        return len(self._free) - self._head

    def allocate(self) -> int:
        if self._head >= len(self._free):
            raise OutOfBlocks(f"all {self.num_blocks} blocks are in use")
        b = self._free[self._head]
        self._head += 1
        self.refcount[b] = 1
        return b

    def share(self, b: int) -> None:
        if self.refcount.get(b, 0) <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.refcount[b] += 1

    def release(self, b: int) -> None:
        rc = self.refcount.get(b, 0)
        if rc <= 0:
            raise ValueError(f"block {b} is not allocated")
        if rc == 1:
            del self.refcount[b]
            self._free.append(b)
        else:
            self.refcount[b] = rc - 1


@dataclass
class SeqState:
    blocks: List[int] = field(default_factory=list)
    num_tokens: int = 0


class BlockManager:
    """Per-sequence block tables over one BlockPool."""

    def __init__(self, block_size: int, pool: BlockPool):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.block_size = block_size
        self.pool = pool
        self.seqs: Dict[int, SeqState] = {}

    # -- sequence life cycle ------------------------------------------------
    def add_sequence(self, seq_id: int, num_tokens: int) -> List[int]:
        """Map ceil(num_tokens / block_size) fresh blocks for a prompt."""
        if seq_id in self.seqs:
            raise ValueError(f"sequence {seq_id} exists")
        nblk = -(-num_tokens // self.block_size)
        st = SeqState([self.pool.allocate() for _ in range(nblk)], num_tokens)
        self.seqs[seq_id] = st
        return list(st.blocks)

    def fork(self, parent: int, child: int) -> None:
        """The child maps every block of the parent (shared, refcount + 1)."""
        if child in self.seqs:
            raise ValueError(f"sequence {child} exists")
        p = self.seqs[parent]
        for b in p.blocks:
            self.pool.share(b)
        self.seqs[child] = SeqState(list(p.blocks), p.num_tokens)

    def free_sequence(self, seq_id: int) -> None:
        for b in self.seqs.pop(seq_id).blocks:
            self.pool.release(b)

    # -- writes ---------------------------------------------------------------
    def make_private(self, seq_id: int, logical: int) -> Optional[Tuple[int, int]]:
        """Copy-on-write of one logical block: if another sequence still maps
        its physical block, map a fresh block here and return the
        (src, dst) copy the cache needs; otherwise return None."""
        st = self.seqs[seq_id]
        old = st.blocks[logical]
        if self.pool.refcount[old] == 1:
            return None
        new = self.pool.allocate()
        self.pool.release(old)
        st.blocks[logical] = new
        return (old, new)

    def append_slot(self, seq_id: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token.

        Returns (slot, copy) where copy is the (src, dst) block copy that has
        to happen before the write, or None."""
        st = self.seqs[seq_id]
        off = st.num_tokens % self.block_size
        copy = None
        if off == 0:
            st.blocks.append(self.pool.allocate())
        else:
            copy = self.make_private(seq_id, len(st.blocks) - 1)
        st.num_tokens += 1
        return st.blocks[-1] * self.block_size + off, copy

    # -- views ----------------------------------------------------------------
    def table(self, seq_id: int) -> List[int]:
        return list(self.seqs[seq_id].blocks)

    def slot_of(self, seq_id: int, t: int) -> int:
        st = self.seqs[seq_id]
        if not 0 <= t < st.num_tokens:
            raise IndexError(t)
        return st.blocks[t // self.block_size] * self.block_size + t % self.block_size

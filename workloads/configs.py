"""The five decode workloads and their seeded synthetic inputs.

No trained weights or request traces are used: q, k and v are drawn from a
seeded N(0, 1) and only the shapes, lengths and sharing patterns follow the
workloads the pages measure (LLaMA-7B-shaped heads, 32 x 128, in
"在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战" §1 and §3.3 and in the
l189.com article www.l189.com/news/180929 §2.1; Llama2-13B, 40 x 128, and
2048-token texts in l189.com §4; block sizes 16 and 32 in l189.com §4).

This module makes inputs only.  It holds none of the kernels' arithmetic; the
one number conversion it does (N(0,1) samples to the stored formats) is a
library cast (torch), used by both sides as given bytes.

Draw order per case, from seed = 423 + config index (NumPy PCG64 for the
index inputs, a torch generator for the tensors): context lengths (and
shared-prefix tails), the permutation that places physical blocks, the fp8
scales, then the tensors q, key, value, k_cache, v_cache.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from .blocks import BlockManager, BlockPool

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.uint8,
               "i8": torch.int8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1, "i8": 1}
# raw-bit views used to hand tensors to the oracle
BITS_TORCH = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16, "e4m3": torch.uint8, "i8": torch.uint8}
BITS_NUMPY = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8, "i8": np.uint8}
SCALED_FORMATS = ("e4m3", "i8")
E4M3_NAN_BYTE = 0x7F
I8_POISON = -128             # never stored by the quantiser (range is [-127, 127])


@dataclass(frozen=True)
class Config:
    index: int                 # 1..5
    name: str
    S: int                     # running sequences
    H: int                     # heads (KV heads = query heads)
    D: int                     # head size
    BS: int                    # block size (tokens per physical block)
    q_dtype: str
    cache_dtype: str
    ctx_dist: str              # "uniform" | "loguniform" | "shared"
    ctx_lo: int
    ctx_hi: int
    MB: int                    # block-table width (max blocks per sequence)
    NB_fixed: Optional[int] = None   # pool size when the workload fixes it
    # shared-prefix workloads: groups of group_size sequences share a prefix
    groups: int = 0
    group_size: int = 0
    prefix_tokens: int = 0
    cow: str = ""              # "last_shared": copy the last shared block for
    #                            every writer before the append; "on_write":
    #                            copy only when the append writes a shared block
    scale_lo: float = 1.0      # 8-bit pools: scale range
    scale_hi: float = 1.0
    head_scales: bool = False  # 8-bit pools: one scale per head (else one per pool)

    @property
    def seed(self) -> int:
        return 423 + self.index


CONFIGS = {
    1: Config(1, "tiny-f32", S=4, H=4, D=64, BS=16, q_dtype="f32", cache_dtype="f32",
              ctx_dist="uniform", ctx_lo=1, ctx_hi=100, MB=7, NB_fixed=64),
    2: Config(2, "llama7b-layer-f16", S=16, H=32, D=128, BS=16, q_dtype="f16", cache_dtype="f16",
              ctx_dist="uniform", ctx_lo=50, ctx_hi=178, MB=12, NB_fixed=223),
    3: Config(3, "llama2-13b-longctx-bf16", S=64, H=40, D=128, BS=16, q_dtype="bf16", cache_dtype="bf16",
              ctx_dist="uniform", ctx_lo=1536, ctx_hi=2048, MB=128),
    4: Config(4, "shared-prefix-cow-f16", S=64, H=32, D=128, BS=16, q_dtype="f16", cache_dtype="f16",
              ctx_dist="shared", ctx_lo=1, ctx_hi=256, MB=49,
              groups=8, group_size=8, prefix_tokens=512, cow="last_shared"),
    5: Config(5, "fp8-e4m3-kv", S=256, H=32, D=128, BS=32, q_dtype="f16", cache_dtype="e4m3",
              ctx_dist="loguniform", ctx_lo=128, ctx_hi=4096, MB=128,
              scale_lo=0.01, scale_hi=0.1),
    # INT8 KV, the other 8-bit format the pages list: the fp8 workload's
    # shape, with scales that put +-127 * scale at about 4 standard deviations
    6: Config(6, "int8-kv", S=256, H=32, D=128, BS=32, q_dtype="f16", cache_dtype="i8",
              ctx_dist="loguniform", ctx_lo=128, ctx_hi=4096, MB=128,
              scale_lo=0.03, scale_hi=0.05),
}

# The two 8-bit workloads with one scale per head instead of one per pool
# (k_scale[h], v_scale[h] ~ U[scale_lo, scale_hi] each): the same lengths,
# placement and tensors' draws as the per-pool workloads.
CONFIG_5_HEAD_SCALES = replace(CONFIGS[5], name="fp8-e4m3-kv-head-scales", head_scales=True)
CONFIG_6_HEAD_SCALES = replace(CONFIGS[6], name="int8-kv-head-scales", head_scales=True)

# C4': the append lands inside the shared last prefix block (500-token
# prefix, no tails), so copy-on-write happens because of the write itself.
CONFIG_4_ON_WRITE = replace(CONFIGS[4], name="shared-prefix-cow-on-write-f16", ctx_lo=0, ctx_hi=0,
                            prefix_tokens=500, cow="on_write", MB=32)


@dataclass
class Case:
    cfg: Config
    S: int
    H: int
    D: int
    BS: int
    NB: int
    MB: int
    q_dtype: str
    cache_dtype: str
    scale: float
    k_scale: object                    # 8-bit pools: float, or float32 [H] (one per head)
    v_scale: object
    context_lens: np.ndarray           # int32 [S], includes the appended token
    block_tables: np.ndarray           # int32 [S, MB], padding = poison block id
    slot_mapping: np.ndarray           # int32 [S], slot of each sequence's new token
    copy_pairs: np.ndarray             # int32 [N, 2], (src, dst), applied before the write
    poison_block: int
    q: torch.Tensor                    # [S, H, D] q_dtype
    key: torch.Tensor                  # [S, H, D] q_dtype (the new token's K)
    value: torch.Tensor                # [S, H, D] q_dtype
    k_cache: torch.Tensor              # [NB, H, BS, D] cache dtype (uint8 bytes for e4m3)
    v_cache: torch.Tensor
    pre_tables: List[List[int]] = field(default_factory=list)   # tables before the step
    groups: List[List[int]] = field(default_factory=list)       # sequences sharing a prefix

    @property
    def kv_bytes(self) -> int:
        """K/V bytes a decode over all sequences reads: sum n_s * H * D * 2 * elem."""
        return int(self.context_lens.astype(np.int64).sum()) * self.H * self.D * 2 * ELEM_BYTES[self.cache_dtype]

    @property
    def unique_kv_bytes(self) -> int:
        """K/V bytes of distinct (physical block, row) pairs read (shared prefixes once)."""
        seen = set()
        for s in range(self.S):
            n = int(self.context_lens[s])
            for t in range(n):
                seen.add((int(self.block_tables[s, t // self.BS]), t % self.BS))
        return len(seen) * self.H * self.D * 2 * ELEM_BYTES[self.cache_dtype]

    def to(self, device) -> "Case":
        c = replace(self)
        for name in ("q", "key", "value", "k_cache", "v_cache"):
            setattr(c, name, getattr(self, name).to(device))
        return c


def draw_context_lens(cfg: Config, rng: np.random.Generator, S: int) -> np.ndarray:
    if cfg.ctx_dist == "uniform":
        return rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=S).astype(np.int32)
    if cfg.ctx_dist == "loguniform":
        u = rng.uniform(math.log(cfg.ctx_lo), math.log(cfg.ctx_hi + 1), size=S)
        return np.minimum(cfg.ctx_hi, np.floor(np.exp(u))).astype(np.int32)
    raise ValueError(cfg.ctx_dist)


def _nan_fill_value(dtype: str):
    if dtype == "e4m3":
        return E4M3_NAN_BYTE
    if dtype == "i8":
        return I8_POISON
    return float("nan")


def _randn_pool(shape, cfg_dtype, scale_for_fp8, gen, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if np.ndim(scale_for_fp8):                   # one scale per head: [H] -> [1, H, 1, 1]
        scale_for_fp8 = torch.as_tensor(np.asarray(scale_for_fp8, np.float32), device=device).view(1, -1, 1, 1)
    if cfg_dtype == "e4m3":
        # stored byte = fp8(x / scale), saturated to the largest finite value
        y = (x / scale_for_fp8).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        return y.view(torch.uint8)
    if cfg_dtype == "i8":
        # stored byte = round(x / scale), saturated to [-127, 127]
        return torch.round(x / scale_for_fp8).clamp_(-127.0, 127.0).to(torch.int8)
    return x.to(TORCH_DTYPE[cfg_dtype])


def make_case(cfg: Config, device="cpu", S: Optional[int] = None, H: Optional[int] = None,
              context_lens: Optional[Sequence[int]] = None, seed: Optional[int] = None,
              NB_slack: float = 1.25) -> Case:
    """Build one seeded decode step of workload ``cfg``.

    Before the step every sequence holds n_s - 1 tokens in the cache; the
    step appends token n_s - 1 (its slot in ``slot_mapping``) and then attends
    over all n_s tokens.  ``S``/``H`` shrink the workload for quick oracle
    runs; ``context_lens`` pins the lengths (edge cases).
    """
    S = cfg.S if S is None else S
    H = cfg.H if H is None else H
    seed = cfg.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    BS = cfg.BS

    # ---- 1. lengths ---------------------------------------------------------
    groups: List[List[int]] = []
    if cfg.ctx_dist == "shared":
        gs = cfg.group_size
        ngroups = max(1, S // gs)
        S = ngroups * gs
        if cfg.ctx_hi > 0:
            tails = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=S).astype(np.int64)
        else:
            tails = np.zeros(S, dtype=np.int64)
        n_pre = cfg.prefix_tokens + tails
        groups = [list(range(g * gs, (g + 1) * gs)) for g in range(ngroups)]
    else:
        if context_lens is not None:
            n_post = np.asarray(context_lens, dtype=np.int64)
            S = n_post.size
        else:
            n_post = draw_context_lens(cfg, rng, S).astype(np.int64)
        if (n_post < 1).any():
            raise ValueError("a decode step appends one token, so every context length is >= 1")
        n_pre = n_post - 1
    MB = cfg.MB
    if context_lens is not None:
        MB = max(MB, int(-(-int(np.max(context_lens)) // BS)))

    # ---- 2. pool size and placement ----------------------------------------
    blocks_post = [-(-int(n + 1) // BS) for n in n_pre]
    if cfg.ctx_dist == "shared":
        prefix_blocks = -(-cfg.prefix_tokens // BS)
        need = len(groups) * prefix_blocks + sum(max(0, b - prefix_blocks) for b in blocks_post)
        copies = len(groups) * (cfg.group_size - 1)
        NB = int(math.ceil(NB_slack * need)) + copies + 1
    elif cfg.NB_fixed is not None and S == cfg.S:
        NB = cfg.NB_fixed
    else:
        NB = int(math.ceil(NB_slack * sum(blocks_post))) + 1
    perm = rng.permutation(NB)

    # ---- 3. 8-bit pool scales -----------------------------------------------
    if cfg.cache_dtype in SCALED_FORMATS and cfg.head_scales:
        k_scale = rng.uniform(cfg.scale_lo, cfg.scale_hi, size=H).astype(np.float32)
        v_scale = rng.uniform(cfg.scale_lo, cfg.scale_hi, size=H).astype(np.float32)
    elif cfg.cache_dtype in SCALED_FORMATS:
        k_scale = float(np.float32(rng.uniform(cfg.scale_lo, cfg.scale_hi)))
        v_scale = float(np.float32(rng.uniform(cfg.scale_lo, cfg.scale_hi)))
    else:
        k_scale = v_scale = 1.0
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))

    # ---- block bookkeeping: history, then the step ---------------------------
    pool = BlockPool(NB, perm)
    poison = pool.allocate()          # never mapped by a sequence; NaN-filled
    bm = BlockManager(BS, pool)
    if cfg.ctx_dist == "shared":
        for grp in groups:
            bm.add_sequence(grp[0], cfg.prefix_tokens)
            for s in grp[1:]:
                bm.fork(grp[0], s)
        for s in range(S):
            for _ in range(int(tails[s])):
                bm.append_slot(s)
    else:
        for s in range(S):
            bm.add_sequence(s, int(n_pre[s]))
    pre_tables = [bm.table(s) for s in range(S)]
    pre_tokens = [bm.seqs[s].num_tokens for s in range(S)]

    pairs: List[Tuple[int, int]] = []
    slots = np.empty(S, dtype=np.int32)
    for s in range(S):
        if cfg.cow == "last_shared":
            last_shared = -(-cfg.prefix_tokens // BS) - 1
            cp = bm.make_private(s, last_shared)
            if cp is not None:
                pairs.append(cp)
        slot, cp = bm.append_slot(s)
        if cp is not None:
            pairs.append(cp)
        slots[s] = slot
    n_post = np.array([bm.seqs[s].num_tokens for s in range(S)], dtype=np.int32)
    if int(n_post.max()) > MB * BS:
        raise ValueError("context longer than the block table allows")
    tables = np.full((S, MB), poison, dtype=np.int32)
    for s in range(S):
        t = bm.table(s)
        tables[s, : len(t)] = t

    # ---- 4. tensors ----------------------------------------------------------
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    qd = TORCH_DTYPE[cfg.q_dtype]
    q = torch.randn((S, H, cfg.D), generator=gen, device=device, dtype=torch.float32).to(qd)
    key = torch.randn((S, H, cfg.D), generator=gen, device=device, dtype=torch.float32).to(qd)
    value = torch.randn((S, H, cfg.D), generator=gen, device=device, dtype=torch.float32).to(qd)
    shape = (NB, H, BS, cfg.D)
    k_cache = _randn_pool(shape, cfg.cache_dtype, k_scale, gen, device)
    v_cache = _randn_pool(shape, cfg.cache_dtype, v_scale, gen, device)

    # NaN in everything no sequence holds before the step: free blocks (the
    # fresh blocks the step maps, the copy destinations), the poison block,
    # and the unfilled slots of each sequence's last block.
    nanv = _nan_fill_value(cfg.cache_dtype)
    mapped = np.zeros(NB, dtype=bool)
    for t in pre_tables:
        mapped[t] = True
    unmapped = torch.from_numpy(np.nonzero(~mapped)[0]).to(device)
    k_cache[unmapped] = nanv
    v_cache[unmapped] = nanv
    for s in range(S):
        t, n = pre_tables[s], pre_tokens[s]
        if t and n % BS:
            k_cache[t[-1], :, n % BS:, :] = nanv
            v_cache[t[-1], :, n % BS:, :] = nanv

    return Case(cfg=cfg, S=S, H=H, D=cfg.D, BS=BS, NB=NB, MB=MB, q_dtype=cfg.q_dtype,
                cache_dtype=cfg.cache_dtype, scale=scale, k_scale=k_scale, v_scale=v_scale,
                context_lens=n_post, block_tables=tables, slot_mapping=slots,
                copy_pairs=np.array(pairs, dtype=np.int32).reshape(-1, 2), poison_block=poison,
                q=q, key=key, value=value, k_cache=k_cache, v_cache=v_cache,
                pre_tables=pre_tables, groups=groups)


def bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Host NumPy copy of a tensor's raw bits in the oracle's convention."""
    return t.detach().contiguous().view(BITS_TORCH[dtype]).cpu().numpy().view(BITS_NUMPY[dtype])


# ---------------------------------------------------------------------------
# prompt (multi-query) workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefillConfig:
    """A batch of sequences, each with q_s new tokens (a prompt, or the part
    of one past tokens already cached) that are written to the cache and then
    attend causally over everything the sequence holds."""
    index: int
    name: str
    S: int
    H: int
    D: int
    BS: int
    dtype: str                 # q, new K/V and output format
    new_lo: int                # new tokens per sequence ~ U{new_lo..new_hi}
    new_hi: int
    cached_lo: int = 0         # tokens cached before the step ~ U{cached_lo..cached_hi}
    cached_hi: int = 0
    groups: int = 0            # groups of group_size sequences share their cached prefix
    group_size: int = 0
    prefix_tokens: int = 0
    cache_dtype: str = ""      # pool format: "" = dtype, or "e4m3" / "i8" with per-pool scales
    scale_lo: float = 0.01     # 8-bit pools: k_scale, v_scale ~ U[scale_lo, scale_hi]
    scale_hi: float = 0.1
    head_scales: bool = False  # 8-bit pools: one scale per head (else one per pool)

    @property
    def pool_dtype(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def seed(self) -> int:
        return 523 + self.index


PREFILL_CONFIGS = {
    1: PrefillConfig(1, "tiny-prefill-f16", S=5, H=4, D=64, BS=16, dtype="f16", new_lo=1, new_hi=100,
                     cached_lo=0, cached_hi=40),
    2: PrefillConfig(2, "llama7b-prompts-f16", S=16, H=32, D=128, BS=16, dtype="f16", new_lo=40, new_hi=60),
    3: PrefillConfig(3, "llama2-13b-long-prompts-bf16", S=16, H=40, D=128, BS=16, dtype="bf16",
                     new_lo=1536, new_hi=2048),
    4: PrefillConfig(4, "shared-prefix-prompts-f16", S=64, H=32, D=128, BS=16, dtype="f16", new_lo=1, new_hi=256,
                     groups=8, group_size=8, prefix_tokens=512),
}


@dataclass
class PrefillCase:
    cfg: PrefillConfig
    S: int
    H: int
    D: int
    BS: int
    NB: int
    MB: int
    dtype: str
    scale: float
    context_lens: np.ndarray           # int32 [S]: tokens held after the step
    q_lens: np.ndarray                 # int32 [S]: new tokens
    cu_q_lens: np.ndarray              # int32 [S + 1]
    block_tables: np.ndarray           # int32 [S, MB], padding = poison block id
    slot_mapping: np.ndarray           # int32 [Tq], slot of every new token
    copy_pairs: np.ndarray             # int32 [N, 2] copies before the write
    poison_block: int
    q: torch.Tensor                    # [Tq, H, D]
    key: torch.Tensor                  # [Tq, H, D] the new tokens' K
    value: torch.Tensor
    k_cache: torch.Tensor              # [NB, H, BS, D] pool format
    v_cache: torch.Tensor
    cache_dtype: str = ""              # pool format (the q format when empty)
    k_scale: object = 1.0              # 8-bit pools: value = byte * scale (float, or float32 [H] per head)
    v_scale: object = 1.0

    @property
    def pool_dtype(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def Tq(self) -> int:
        return int(self.cu_q_lens[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.S else 0

    @property
    def attn_pairs(self) -> int:
        """(query, visible key) pairs over all sequences, per head."""
        n = self.context_lens.astype(np.int64)
        q = self.q_lens.astype(np.int64)
        return int((q * (n - q) + q * (q + 1) // 2).sum())

    @property
    def flops(self) -> int:
        """Multiply-adds of q.k and p.v counted as 2 flops each: 4 * D per pair and head."""
        return 4 * self.D * self.H * self.attn_pairs

    def to(self, device) -> "PrefillCase":
        c = replace(self)
        for name in ("q", "key", "value", "k_cache", "v_cache"):
            setattr(c, name, getattr(self, name).to(device))
        return c


def make_prefill_case(cfg: PrefillConfig, device="cpu", S: Optional[int] = None, H: Optional[int] = None,
                      q_lens: Optional[Sequence[int]] = None, cached: Optional[Sequence[int]] = None,
                      seed: Optional[int] = None, NB_slack: float = 1.25) -> PrefillCase:
    """Build one seeded prompt step of workload ``cfg``: sequence s holds
    cached[s] tokens (its shared prefix, if grouped), q_lens[s] new tokens
    get slots by the append rule (copy-on-write where a shared block is
    written), and the step writes them and attends over all of them.
    Draw order: cached lengths, new lengths, placement, then q, key, value
    and the two pools."""
    S = cfg.S if S is None else S
    H = cfg.H if H is None else H
    seed = cfg.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    BS = cfg.BS

    groups: List[List[int]] = []
    if cfg.groups:
        gs = cfg.group_size
        S = max(1, S // gs) * gs
        groups = [list(range(g * gs, (g + 1) * gs)) for g in range(S // gs)]
        n_cached = np.full(S, cfg.prefix_tokens, dtype=np.int64)
    elif cached is not None:
        n_cached = np.asarray(cached, dtype=np.int64)
        S = n_cached.size
    else:
        n_cached = rng.integers(cfg.cached_lo, cfg.cached_hi + 1, size=S).astype(np.int64)
    if q_lens is not None:
        n_new = np.asarray(q_lens, dtype=np.int64)
        if n_new.size != S:
            raise ValueError("q_lens must give one length per sequence")
    else:
        n_new = rng.integers(cfg.new_lo, cfg.new_hi + 1, size=S).astype(np.int64)

    if groups:
        prefix_blocks = -(-cfg.prefix_tokens // BS)
        need = len(groups) * prefix_blocks + sum(-(-int(n + cfg.prefix_tokens) // BS) - cfg.prefix_tokens // BS
                                                 for n in n_new)
    else:
        need = sum(-(-int(c + n) // BS) for c, n in zip(n_cached, n_new))
    NB = int(math.ceil(NB_slack * need)) + 1
    perm = rng.permutation(NB)
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    pdt = cfg.pool_dtype
    k_scale = v_scale = 1.0
    if pdt in ("e4m3", "i8") and cfg.head_scales:
        k_scale = rng.uniform(cfg.scale_lo, cfg.scale_hi, size=H).astype(np.float32)
        v_scale = rng.uniform(cfg.scale_lo, cfg.scale_hi, size=H).astype(np.float32)
    elif pdt in ("e4m3", "i8"):                 # drawn after the placement: 16-bit workloads draw as before
        k_scale = float(np.float32(rng.uniform(cfg.scale_lo, cfg.scale_hi)))
        v_scale = float(np.float32(rng.uniform(cfg.scale_lo, cfg.scale_hi)))

    pool = BlockPool(NB, perm)
    poison = pool.allocate()
    bm = BlockManager(BS, pool)
    if groups:
        for grp in groups:
            bm.add_sequence(grp[0], cfg.prefix_tokens)
            for s in grp[1:]:
                bm.fork(grp[0], s)
    else:
        for s in range(S):
            bm.add_sequence(s, int(n_cached[s]))
    pre_tables = [bm.table(s) for s in range(S)]
    pairs: List[Tuple[int, int]] = []
    slots = []
    for s in range(S):
        for _ in range(int(n_new[s])):
            slot, cp = bm.append_slot(s)
            if cp is not None:
                pairs.append(cp)
            slots.append(slot)
    n_post = np.array([bm.seqs[s].num_tokens for s in range(S)], dtype=np.int32)
    MB = max(1, max(len(bm.table(s)) for s in range(S)))
    tables = np.full((S, MB), poison, dtype=np.int32)
    for s in range(S):
        t = bm.table(s)
        tables[s, : len(t)] = t
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n_new)

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = TORCH_DTYPE[cfg.dtype]
    Tq = int(cu[-1])
    q = torch.randn((Tq, H, cfg.D), generator=gen, device=device, dtype=torch.float32).to(dt)
    key = torch.randn((Tq, H, cfg.D), generator=gen, device=device, dtype=torch.float32).to(dt)
    value = torch.randn((Tq, H, cfg.D), generator=gen, device=device, dtype=torch.float32).to(dt)
    shape = (NB, H, BS, cfg.D)
    k_cache = _randn_pool(shape, pdt, k_scale, gen, device)
    v_cache = _randn_pool(shape, pdt, v_scale, gen, device)

    # NaN (8-bit: the poison byte) wherever no cached token lives before the step
    nanv = _nan_fill_value(pdt)
    mapped = np.zeros(NB, dtype=bool)
    for t in pre_tables:
        mapped[t] = True
    unmapped = torch.from_numpy(np.nonzero(~mapped)[0]).to(device)
    k_cache[unmapped] = nanv
    v_cache[unmapped] = nanv
    for s in range(S):
        t, n = pre_tables[s], int(n_cached[s])
        if t and n % BS:
            k_cache[t[-1], :, n % BS:, :] = nanv
            v_cache[t[-1], :, n % BS:, :] = nanv

    return PrefillCase(cfg=cfg, S=S, H=H, D=cfg.D, BS=BS, NB=NB, MB=MB, dtype=cfg.dtype, scale=scale,
                       context_lens=n_post, q_lens=n_new.astype(np.int32), cu_q_lens=cu, block_tables=tables,
                       slot_mapping=np.array(slots, dtype=np.int32),
                       copy_pairs=np.array(pairs, dtype=np.int32).reshape(-1, 2), poison_block=poison,
                       q=q, key=key, value=value, k_cache=k_cache, v_cache=v_cache,
                       cache_dtype="" if pdt == cfg.dtype else pdt, k_scale=k_scale, v_scale=v_scale)

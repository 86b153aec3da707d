"""Seeded random block copies and block gathers against the oracle (GPU).

Pools of random bytes in every element format and head size; copy pairs
drawn at random (distinct destinations that are not sources, as the
operation requires), tables drawn at random (blocks may repeat across
sequences, as with shared prefixes) with lengths from 0 to the table's
capacity.  Both operations are bit copies, so the results must equal the
oracle's bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import require_gpu

pytestmark = pytest.mark.gpu

FORMATS = ["f32", "f16", "bf16", "e4m3", "i8"]


def _pool(rng, NB, H, BS, D, fmt, gen):
    eb = W.ELEM_BYTES[fmt]
    raw = torch.randint(0, 256, (NB, H, BS, D * eb), dtype=torch.uint8, generator=gen)
    return raw.view(W.TORCH_DTYPE[fmt]).cuda()


def _case(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = torch.Generator().manual_seed(seed)
    D = int(rng.choice([64, 80, 96, 128, 256]))
    BS = int(rng.choice([16, 32]))
    fmt = FORMATS[int(rng.integers(len(FORMATS)))]
    NB, H = int(rng.integers(8, 160)), int(rng.integers(1, 5))
    return rng, gen, D, BS, fmt, NB, H


@pytest.mark.parametrize("seed", range(10))
def test_random_block_copies(seed):
    pkv = require_gpu()
    rng, gen, D, BS, fmt, NB, H = _case(6230 + seed)
    k, v = _pool(rng, NB, H, BS, D, fmt, gen), _pool(rng, NB, H, BS, D, fmt, gen)
    perm = rng.permutation(NB)
    N = int(rng.integers(1, NB // 2 + 1))
    dst = perm[:N]
    src = rng.choice(perm[N:], N)                       # sources may repeat, never a destination
    pairs = np.stack([src, dst], 1).astype(np.int32)
    print(f"[copy fuzz {seed}] {fmt} NB={NB} H={H} BS={BS} D={D} pairs={N}", flush=True)
    kb, vb = W.bits(k, fmt), W.bits(v, fmt)
    pkv.copy_blocks(k, v, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    ko, vo = oracle.copy_blocks(kb, vb, pairs)
    assert np.array_equal(W.bits(k, fmt), ko) and np.array_equal(W.bits(v, fmt), vo)


@pytest.mark.parametrize("seed", range(10))
def test_random_block_gathers(seed):
    pkv = require_gpu()
    rng, gen, D, BS, fmt, NB, H = _case(7230 + seed)
    k, v = _pool(rng, NB, H, BS, D, fmt, gen), _pool(rng, NB, H, BS, D, fmt, gen)
    S, MB = int(rng.integers(1, 9)), int(rng.integers(1, 12))
    tables = rng.integers(0, NB, (S, MB)).astype(np.int32)
    lens = rng.integers(0, MB * BS + 1, S).astype(np.int32)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    print(f"[gather fuzz {seed}] {fmt} NB={NB} H={H} BS={BS} D={D} S={S} MB={MB} lens={lens.tolist()}", flush=True)
    total = max(int(cu[-1]), 1)
    ko = torch.empty((total, H, D), dtype=k.dtype, device="cuda")
    vo = torch.empty_like(ko)
    pkv.gather_kv(ko, vo, torch.from_numpy(cu).cuda(), k, v, torch.from_numpy(tables).cuda(),
                  torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    ke, ve, _ = oracle.gather_kv(W.bits(k, fmt), W.bits(v, fmt), tables, lens)
    n = int(cu[-1])
    assert np.array_equal(W.bits(ko, fmt)[:n], ke) and np.array_equal(W.bits(vo, fmt)[:n], ve)

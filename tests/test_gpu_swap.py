"""GPU: block swap between the GPU pools and a pinned host swap space
(pkv_swap_blocks) against the oracle, bit for bit.

Swap-out moves sequences' blocks to host memory; swap-in brings them back,
possibly to other physical blocks.  The pools must match the oracle's swap of
the same pre-state exactly, and a decode over the swapped-in blocks (tables
renamed to match) must equal the decode before the swap bit for bit.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import require_gpu

pytestmark = pytest.mark.gpu


def _b(t, fmt):
    return W.bits(t, fmt)


def test_swap_out_then_in_elsewhere():
    pkv = require_gpu()
    case = W.make_case(W.CONFIGS[2], device="cuda")
    fmt = case.cache_dtype
    pkv.reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                          torch.from_numpy(case.slot_mapping).cuda())
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    before = torch.empty_like(case.q)
    pkv.paged_attention_decode(before, case.q, case.k_cache, case.v_cache, bt, cl, case.scale)
    torch.cuda.synchronize()

    # swap out the blocks of sequences 3, 7 and 11 to the host
    victims = [3, 7, 11]
    out_ids = []
    for s in victims:
        out_ids += [int(b) for b in case.block_tables[s, : -(-int(case.context_lens[s]) // case.BS)]]
    M = len(out_ids)
    host_k = torch.full((M + 3,) + tuple(case.k_cache.shape[1:]), float("nan"), dtype=case.k_cache.dtype).pin_memory()
    host_v = host_k.clone().pin_memory()
    out_pairs = torch.tensor([[b, i] for i, b in enumerate(out_ids)], dtype=torch.int32).cuda()
    gk_pre, gv_pre = _b(case.k_cache, fmt), _b(case.v_cache, fmt)
    hk_pre, hv_pre = _b(host_k, fmt), _b(host_v, fmt)
    pkv.swap_blocks(host_k, host_v, case.k_cache, case.v_cache, out_pairs)
    torch.cuda.synchronize()
    wk, wv = oracle.swap_blocks(gk_pre, gv_pre, hk_pre, hv_pre, out_pairs.cpu().numpy())
    assert np.array_equal(_b(host_k, fmt), wk) and np.array_equal(_b(host_v, fmt), wv), "swap-out differs"

    # the GPU blocks are reused (poisoned here); bring the sequences back to fresh blocks
    used = set(int(b) for s in range(case.S)
               for b in case.block_tables[s, : -(-int(case.context_lens[s]) // case.BS)])
    fresh = [b for b in range(case.NB) if b not in used and b != case.poison_block][:M]
    assert len(fresh) == M
    idx = torch.tensor(out_ids, device="cuda")
    case.k_cache[idx] = float("nan")
    case.v_cache[idx] = float("nan")
    gk_mid, gv_mid = _b(case.k_cache, fmt), _b(case.v_cache, fmt)
    in_pairs = torch.tensor([[i, b] for i, b in enumerate(fresh)], dtype=torch.int32).pin_memory()
    pkv.swap_blocks(case.k_cache, case.v_cache, host_k, host_v, in_pairs)
    torch.cuda.synchronize()
    wk2, wv2 = oracle.swap_blocks(_b(host_k, fmt), _b(host_v, fmt), gk_mid, gv_mid, in_pairs.numpy())
    assert np.array_equal(_b(case.k_cache, fmt), wk2) and np.array_equal(_b(case.v_cache, fmt), wv2), "swap-in differs"

    tables2 = case.block_tables.copy()
    remap = dict(zip(out_ids, fresh))
    for s in victims:
        nb = -(-int(case.context_lens[s]) // case.BS)
        tables2[s, :nb] = [remap[int(b)] for b in case.block_tables[s, :nb]]
    after = torch.empty_like(case.q)
    pkv.paged_attention_decode(after, case.q, case.k_cache, case.v_cache, torch.from_numpy(tables2).cuda(), cl,
                               case.scale)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.uint8])
def test_swap_formats_and_skipped_pairs(dtype):
    pkv = require_gpu()
    fmt = {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "e4m3"}[dtype]
    g = torch.Generator().manual_seed(9)
    shape = (40, 4, 32, 64)
    if dtype == torch.uint8:
        gk = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
        gv = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
    else:
        gk = torch.randn(shape, generator=g).to(dtype)
        gv = torch.randn(shape, generator=g).to(dtype)
    hk = torch.zeros((9,) + shape[1:], dtype=dtype).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    pairs = np.array([[5, 0], [39, 8], [0, 3], [-1, 2], [7, 9], [12, 4]], dtype=np.int32)   # two skipped
    want_k, want_v = oracle.swap_blocks(_b(gk, fmt), _b(gv, fmt), _b(hk, fmt), _b(hv, fmt),
                                        pairs[[0, 1, 2, 5]])
    gkd, gvd = gk.cuda(), gv.cuda()
    pkv.swap_blocks(hk, hv, gkd, gvd, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_b(hk, fmt), want_k) and np.array_equal(_b(hv, fmt), want_v)


def test_swap_refuses_pageable_host_memory():
    """The C entry point checks every pointer before launching: an ordinary
    (pageable) host buffer is refused with PKV_ERR_INVALID_ARG."""
    pkv = require_gpu()
    lib = pkv.lib()
    shape = (4, 2, 16, 64)
    dev_k = torch.zeros(shape, dtype=torch.float16, device="cuda")
    dev_v = torch.zeros_like(dev_k)
    pageable = np.zeros(int(np.prod(shape)) + 64, dtype=np.float16)
    addr = (pageable.ctypes.data + 15) // 16 * 16
    pairs = torch.tensor([[0, 0]], dtype=torch.int32, device="cuda")
    st = lib.pkv_swap_blocks(ctypes.c_void_p(addr), ctypes.c_void_p(addr), ctypes.c_void_p(dev_k.data_ptr()),
                             ctypes.c_void_p(dev_v.data_ptr()), ctypes.c_void_p(pairs.data_ptr()), 1, 2, 64, 16, 4, 4,
                             pkv.PKV_F16, None)
    assert st == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        pkv.swap_blocks(torch.zeros(shape, dtype=torch.float16), dev_v.cpu(), dev_k, dev_v, pairs)
    torch.cuda.synchronize()

"""GPU: the prompt step that stores its new tokens itself
(pkv_paged_attention_prefill_append).

The fused call must give, bit for bit in the output and in both whole pools,
what the cache write followed by the prompt attention gives on the same
inputs, and it is checked against the oracle.  Cases: every prompt workload
(whole prompts, prompts after a cached shared prefix with copy-on-write),
the tile-boundary shapes of every head and block size, a skipped slot, and
the host-side checks.
"""

import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import require_gpu
from test_gpu_prefill import check, oracle_run, sample

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _pools(pkv, case):
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    if case.copy_pairs.shape[0]:
        pkv.copy_blocks(kc, vc, torch.from_numpy(case.copy_pairs).cuda())
    return kc, vc


def _args(case, slots=None):
    sl = case.slot_mapping if slots is None else slots
    return (torch.from_numpy(sl).cuda(), torch.from_numpy(case.block_tables).cuda(),
            torch.from_numpy(case.context_lens).cuda(), torch.from_numpy(case.cu_q_lens).cuda())


def run_separate(pkv, case, slots=None):
    kc, vc = _pools(pkv, case)
    sl, bt, cl, cu = _args(case, slots)
    pkv.reshape_and_cache(case.key, case.value, kc, vc, sl, case.k_scale, case.v_scale)
    out = torch.full_like(case.q, float("nan"))
    pkv.paged_attention_prefill(out, case.q, kc, vc, bt, cl, cu, case.max_q_len, case.scale, case.k_scale,
                                case.v_scale)
    torch.cuda.synchronize()
    return kc, vc, out


def run_append(pkv, case, slots=None):
    kc, vc = _pools(pkv, case)
    sl, bt, cl, cu = _args(case, slots)
    out = torch.full_like(case.q, float("nan"))
    pkv.paged_attention_prefill_append(out, case.q, case.key, case.value, kc, vc, sl, bt, cl, cu, case.max_q_len,
                                       case.scale, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    return kc, vc, out


def assert_same(a, b, label):
    for name, x, y in zip(("K pool", "V pool", "output"), a, b):
        assert torch.equal(_bits(x), _bits(y)), f"{label}: {name} differs between the fused and the separate calls"


@pytest.mark.parametrize("idx,nsample", [(1, None), (2, None), (3, 2), (4, None)])
def test_prefill_append_workloads(idx, nsample):
    pkv = require_gpu()
    cfg = W.PREFILL_CONFIGS[idx]
    case = W.make_prefill_case(cfg, device="cuda")
    print(f"[prefill append] {cfg.name}: S={case.S} Tq={case.Tq}", flush=True)
    fused = run_append(pkv, case)
    assert_same(fused, run_separate(pkv, case), cfg.name)
    seqs = None if nsample is None else sample(case, nsample)
    o = oracle_run(case, case.k_cache, case.v_cache, seqs)
    err = check(case, fused[0], fused[1], fused[2], o, cfg.name + " (fused)")
    print(f"[prefill append] {cfg.name}: max abs error {err:.3g}", flush=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,BS", [(64, 16), (64, 32), (80, 16), (96, 32), (128, 16), (128, 32), (256, 16)])
def test_prefill_append_tile_boundaries(dtype, D, BS):
    """Lengths around the 32-key tile, the 128-query workgroup tile and the
    block size, with and without a cached prefix, and a sequence with no new
    tokens: the tiles then mix rows from the pools and from key / value."""
    pkv = require_gpu()
    cfg = replace(W.PREFILL_CONFIGS[1], D=D, BS=BS, dtype=dtype, H=2)
    q_lens = [1, 31, 32, 33, 127, 128, 129, 0, 200, 5, 64]
    cached = [0, 0, 0, 0, 0, 1, 15, 9, 17, 300, 64]
    case = W.make_prefill_case(cfg, device="cuda", q_lens=q_lens, cached=cached, seed=78)
    print(f"[prefill append] {dtype} D={D} BS={BS}", flush=True)
    fused = run_append(pkv, case)
    assert_same(fused, run_separate(pkv, case), f"{dtype} D{D} BS{BS}")
    check(case, fused[0], fused[1], fused[2], oracle_run(case, case.k_cache, case.v_cache), f"{dtype} D{D} BS{BS}")


@pytest.mark.parametrize("dtype,D,BS", [("bf16", 128, 16), ("f16", 64, 32)])
def test_prefill_append_first_sequence_after_a_prefix(dtype, D, BS):
    """The batch's first new tokens follow a cached prefix that ends inside a
    32-key tile: that tile's rows before the first new token come from the
    pools and the rest from key / value rows counted from before the start of
    key / value (the tile's row 0 lies before it)."""
    pkv = require_gpu()
    cfg = replace(W.PREFILL_CONFIGS[1], D=D, BS=BS, dtype=dtype, H=3)
    q_lens = [50, 3, 130, 1]
    cached = [9, 45, 33, 31]
    case = W.make_prefill_case(cfg, device="cuda", q_lens=q_lens, cached=cached, seed=79)
    print(f"[prefill append] first sequence after a prefix: {dtype} D={D} BS={BS}", flush=True)
    fused = run_append(pkv, case)
    assert_same(fused, run_separate(pkv, case), f"first after prefix {dtype} D{D} BS{BS}")
    check(case, fused[0], fused[1], fused[2], oracle_run(case, case.k_cache, case.v_cache),
          f"first after prefix {dtype} D{D} BS{BS}")


@pytest.mark.parametrize("cache", ["e4m3", "i8"])
def test_prefill_append_8bit_pools(cache):
    """8-bit pools: the cache write quantises the new tokens, then the prompt
    attention reads them back; bitwise the separate calls, and the oracle."""
    pkv = require_gpu()
    cfg = replace(W.PREFILL_CONFIGS[4], dtype="bf16", cache_dtype=cache)
    case = W.make_prefill_case(cfg, device="cuda", S=16)
    print(f"[prefill append] {cfg.name} bf16/{cache}: S={case.S} Tq={case.Tq}", flush=True)
    fused = run_append(pkv, case)
    assert_same(fused, run_separate(pkv, case), f"{cfg.name} {cache}")
    check(case, fused[0], fused[1], fused[2], oracle_run(case, case.k_cache, case.v_cache), f"{cfg.name} {cache}")


def test_prefill_append_skipped_slot():
    """A negative slot skips that token's write (the pools equal those of the
    cache write with the same slots); the attention still takes the token's
    K/V from key / value, so the output is the one with the token stored."""
    pkv = require_gpu()
    case = W.make_prefill_case(W.PREFILL_CONFIGS[2], device="cuda")
    slots = case.slot_mapping.copy()
    skip = [3, int(case.cu_q_lens[5]) + 7]
    slots[skip] = -1
    print(f"[prefill append] skipped slots at tokens {skip}", flush=True)
    kc, vc, out = run_append(pkv, case, slots)
    ks, vs, _ = run_separate(pkv, case, slots)
    assert torch.equal(_bits(kc), _bits(ks)) and torch.equal(_bits(vc), _bits(vs))
    _, _, out_all = run_append(pkv, case)
    assert torch.equal(_bits(out), _bits(out_all))


def test_prefill_append_status_codes():
    pkv = require_gpu()
    lib = pkv.lib()
    case = W.make_prefill_case(W.PREFILL_CONFIGS[1], device="cuda")
    sl, bt, cl, cu = _args(case)
    out = torch.empty_like(case.q)
    P = ctypes.c_void_p
    code = {"f16": 1, "bf16": 2}[case.dtype]

    def call(key=case.key.data_ptr(), value=case.value.data_ptr(), slots=sl.data_ptr(), S=case.S):
        return lib.pkv_paged_attention_prefill_append(
            P(out.data_ptr()), P(case.q.data_ptr()), P(key), P(value), P(case.k_cache.data_ptr()),
            P(case.v_cache.data_ptr()), P(slots), P(bt.data_ptr()), P(cl.data_ptr()), P(cu.data_ptr()), S, case.Tq,
            case.max_q_len, case.H, case.D, case.BS, case.MB, case.NB, case.scale, code, code, 1.0, 1.0, None)

    assert call(key=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(value=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(slots=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(key=case.key.reshape(-1).view(torch.uint8)[2:].data_ptr()) == pkv.PKV_ERR_INVALID_ARG
    assert call(S=0) == pkv.PKV_OK
    with pytest.raises(ValueError):
        pkv.paged_attention_prefill_append(out, case.q, case.key[:1].contiguous(), case.value, case.k_cache,
                                           case.v_cache, sl, bt, cl, cu, case.max_q_len, case.scale)
    torch.cuda.synchronize()

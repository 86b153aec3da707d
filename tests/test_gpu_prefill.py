"""GPU parity of the multi-query (prompt) step: copy-on-write copies, the cache
write of every new token, then paged_attention_prefill, against the oracle.

Tolerance.  The kernel accumulates in fp32 but rounds each softmax weight to
the operand format of the matrix cores (bf16: 8 significant bits, fp16: 11),
round to nearest, before it multiplies V, and its normaliser sums those same
rounded weights.  8-bit pool values (E4M3, INT8) are converted to the operand
format exactly, and their scales multiply the scores and the output in fp32,
so the same bound holds for them.  (INT8 values enter as byte + 128, and
128 sum(q) and 128 sum(p) come off in fp32; with one fp32 rounding per
16-key matrix instruction that moves the output by at most about
(n / 16) 2^-24 255 v_scale, 1.6e-4 at 2048 keys and scale 0.05, inside the
2e-3 term.)  Each rounded weight is w_t (1 + delta_t) with |delta_t| <= u,
the unit roundoff of the operand format (u = 2^-8 for bf16, 2^-11 for fp16).
With p = softmax, the output is
    sum_t p_t (1 + delta_t) V_t / (1 + sum_s p_s delta_s),
which differs from sum_t p_t V_t = o by
    (sum_t p_t delta_t V_t - o sum_s p_s delta_s) / (1 + sum_s p_s delta_s),
at most u (sum_t p_t |V_t| + |o|) / (1 - u): the numerator's rounding and
the normaliser's.  sum_t p_t |V_t| (the softmax average of |V|) comes from
the oracle run on V with its sign bits cleared.  Each element is allowed
    2e-3 + u (sum_t p_t |V_t| + |o|) / (1 - u) + half an ulp of the output
    format at |o|
(the last term is the output's own rounding, relative 2^-8 or 2^-11).
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import out_f64, require_gpu

pytestmark = pytest.mark.gpu

U_P = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}        # unit roundoff of the weights' operand format
OUT_REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}    # half an ulp of the output format, relative


def abs_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    """Raw bits of |x| for the pool format (the oracle then averages |V|)."""
    if dtype == "i8":
        return np.minimum(np.abs(b.view(np.int8).astype(np.int16)), 127).astype(np.int8).view(np.uint8)
    if dtype == "e4m3":
        return b & np.uint8(0x7F)
    return b & np.uint16(0x7FFF)


def run_gpu(pkv, case: W.PrefillCase, keep_pre=True):
    dev = "cuda"
    c = case if case.k_cache.device.type == "cuda" else case.to(dev)
    k_pre = c.k_cache.clone() if keep_pre else None
    v_pre = c.v_cache.clone() if keep_pre else None
    if case.copy_pairs.shape[0]:
        pkv.copy_blocks(c.k_cache, c.v_cache, torch.from_numpy(case.copy_pairs).to(dev))
    pkv.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, torch.from_numpy(case.slot_mapping).to(dev),
                          case.k_scale, case.v_scale)
    out = torch.full_like(c.q, float("nan"))
    pkv.paged_attention_prefill(out, c.q, c.k_cache, c.v_cache, torch.from_numpy(case.block_tables).to(dev),
                                torch.from_numpy(case.context_lens).to(dev), torch.from_numpy(case.cu_q_lens).to(dev),
                                case.max_q_len, case.scale, case.k_scale, case.v_scale)
    torch.cuda.synchronize()
    return k_pre, v_pre, c.k_cache, c.v_cache, out


def oracle_run(case: W.PrefillCase, k_pre: torch.Tensor, v_pre: torch.Tensor, seqs: Optional[Sequence[int]] = None):
    """The same step in the oracle for ``seqs``: the blocks they map (and the
    copy sources) move to the host, renumbered; returns the mini pools after
    copy + write, the mapped mini ids, their physical ids, the output rows
    and the softmax average of |V| per output element."""
    seqs = list(range(case.S)) if seqs is None else list(seqs)
    BS, dt, pdt = case.BS, case.dtype, case.pool_dtype
    need = set()
    for s in seqs:
        nb = -(-int(case.context_lens[s]) // BS)
        need.update(int(b) for b in case.block_tables[s, :nb])
    mapped_ids = sorted(need)
    pairs = [(int(a), int(b)) for a, b in case.copy_pairs if int(b) in need]
    need.update(a for a, _ in pairs)
    blocks = np.array(sorted(need), dtype=np.int64)
    remap: Dict[int, int] = {int(b): i for i, b in enumerate(blocks)}
    idx = torch.from_numpy(blocks).to(k_pre.device)
    kb = W.bits(k_pre.index_select(0, idx), pdt)
    vb = W.bits(v_pre.index_select(0, idx), pdt)
    mini_pairs = np.array([(remap[a], remap[b]) for a, b in pairs], dtype=np.int64).reshape(-1, 2)
    kb, vb = oracle.copy_blocks(kb, vb, mini_pairs)
    rows: List[int] = []
    for s in seqs:
        rows.extend(range(int(case.cu_q_lens[s]), int(case.cu_q_lens[s + 1])))
    rows_t = torch.as_tensor(rows, dtype=torch.long)
    sl = case.slot_mapping[rows].astype(np.int64)
    mini_slots = np.array([remap[int(x) // BS] * BS + int(x) % BS for x in sl], dtype=np.int64)
    key = W.bits(case.key.index_select(0, rows_t.to(case.key.device)), dt)
    val = W.bits(case.value.index_select(0, rows_t.to(case.value.device)), dt)
    kb, vb = oracle.reshape_and_cache(key, val, kb, vb, mini_slots, dt, pdt, case.k_scale, case.v_scale)
    tables = np.zeros((len(seqs), case.MB), dtype=np.int64)
    for i, s in enumerate(seqs):
        nb = -(-int(case.context_lens[s]) // BS)
        tables[i, :nb] = [remap[int(b)] for b in case.block_tables[s, :nb]]
    q = W.bits(case.q.index_select(0, rows_t.to(case.q.device)), dt)
    cu = np.zeros(len(seqs) + 1, dtype=np.int64)
    cu[1:] = np.cumsum([int(case.q_lens[s]) for s in seqs])
    lens = case.context_lens[seqs]
    out = oracle.paged_attention_prefill(q, kb, vb, tables, lens, cu, case.scale, dt, pdt, case.k_scale,
                                         case.v_scale)
    avg_abs_v = oracle.paged_attention_prefill(q, kb, abs_bits(vb, pdt), tables, lens, cu, case.scale, dt, pdt,
                                               case.k_scale, case.v_scale)
    mapped = np.array([remap[b] for b in mapped_ids], dtype=np.int64)
    return dict(rows=rows, blocks=blocks, mapped=mapped, k=kb, v=vb, out=out, avg_abs_v=avg_abs_v)


def check(case: W.PrefillCase, gk, gv, gout, o, label=""):
    idx = torch.from_numpy(o["blocks"][o["mapped"]]).to(gk.device)
    pdt = case.pool_dtype
    assert np.array_equal(W.bits(gk.index_select(0, idx), pdt), o["k"][o["mapped"]]), f"{label}: K pool differs"
    assert np.array_equal(W.bits(gv.index_select(0, idx), pdt), o["v"][o["mapped"]]), f"{label}: V pool differs"
    if not o["rows"]:
        return 0.0
    got = out_f64(gout.index_select(0, torch.as_tensor(o["rows"], device=gout.device)))
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    want = o["out"]
    diff = np.abs(got - want)
    u = U_P[case.dtype]
    bound = 2e-3 + u * (o["avg_abs_v"] + np.abs(want)) / (1.0 - u) + OUT_REL[case.dtype] * np.abs(want)
    bad = diff > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(diff - bound)), diff.shape)
        raise AssertionError(f"{label}: {int(bad.sum())} of {diff.size} elements over the bound; worst at row "
                             f"{o['rows'][i[0]]} head {i[1]} dim {i[2]}: got {got[i]!r} want {want[i]!r} "
                             f"bound {bound[i]:.3g}")
    return float(diff.max())


def sample(case: W.PrefillCase, k: int, seed=0) -> List[int]:
    n = case.q_lens
    pick = {int(np.argmin(n)), int(np.argmax(n))}
    rng = np.random.default_rng(seed)
    for s in rng.permutation(case.S):
        if len(pick) >= min(k, case.S):
            break
        pick.add(int(s))
    return sorted(pick)


@pytest.mark.parametrize("idx,nsample", [(1, None), (2, None), (3, 2), (4, None)])
def test_prefill_workloads_match_oracle(idx, nsample):
    pkv = require_gpu()
    cfg = W.PREFILL_CONFIGS[idx]
    case = W.make_prefill_case(cfg, device="cuda")
    print(f"prefill workload {cfg.name}: S={case.S} Tq={case.Tq} max_q={case.max_q_len}", flush=True)
    k_pre, v_pre, gk, gv, gout = run_gpu(pkv, case)
    seqs = None if nsample is None else sample(case, nsample)
    o = oracle_run(case, k_pre, v_pre, seqs)
    err = check(case, gk, gv, gout, o, cfg.name)
    print(f"{cfg.name}: max abs error {err:.3g}", flush=True)
    if seqs is not None:
        assert torch.isfinite(gout.float()).all(), "non-finite output outside the sampled sequences"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,BS", [(64, 16), (64, 32), (80, 16), (96, 32), (128, 16), (128, 32), (256, 16)])
def test_prefill_tile_boundaries(dtype, D, BS):
    """Lengths around the 32-key tile, the 128-query workgroup tile and the
    block size, with and without a cached prefix, and a sequence with no new
    tokens."""
    pkv = require_gpu()
    from dataclasses import replace
    cfg = replace(W.PREFILL_CONFIGS[1], D=D, BS=BS, dtype=dtype, H=2)
    q_lens = [1, 31, 32, 33, 127, 128, 129, 0, 200, 5, 64]
    cached = [0, 0, 0, 0, 0, 1, 15, 9, 17, 300, 64]
    case = W.make_prefill_case(cfg, device="cuda", q_lens=q_lens, cached=cached, seed=77)
    k_pre, v_pre, gk, gv, gout = run_gpu(pkv, case)
    err = check(case, gk, gv, gout, oracle_run(case, k_pre, v_pre), f"{dtype} D{D} BS{BS}")
    print(f"{dtype} D={D} BS={BS}: max abs error {err:.3g}", flush=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("cache", ["e4m3", "i8"])
@pytest.mark.parametrize("idx,nsample", [(2, None), (4, 4)])
def test_prefill_8bit_pools_match_oracle(dtype, cache, idx, nsample):
    """Prompts over E4M3 and INT8 pools with per-pool scales (the new tokens
    quantised by the cache write, the cached context read back through the
    tables), whole prompts and prompts after a shared cached prefix."""
    pkv = require_gpu()
    from dataclasses import replace
    cfg = replace(W.PREFILL_CONFIGS[idx], dtype=dtype, cache_dtype=cache)
    case = W.make_prefill_case(cfg, device="cuda")
    print(f"prefill {cfg.name} {dtype}/{cache}: S={case.S} Tq={case.Tq} k_scale={case.k_scale:.4g} "
          f"v_scale={case.v_scale:.4g}", flush=True)
    k_pre, v_pre, gk, gv, gout = run_gpu(pkv, case)
    seqs = None if nsample is None else sample(case, nsample)
    err = check(case, gk, gv, gout, oracle_run(case, k_pre, v_pre, seqs), f"{cfg.name} {dtype}/{cache}")
    print(f"{cfg.name} {dtype}/{cache}: max abs error {err:.3g}", flush=True)


@pytest.mark.parametrize("cache", ["e4m3", "i8"])
@pytest.mark.parametrize("D,BS", [(64, 16), (80, 32), (96, 16), (128, 16), (128, 32), (256, 16)])
def test_prefill_8bit_tile_boundaries(cache, D, BS):
    """The tile-boundary shapes over 8-bit pools: the staged loads cover half
    a round (D = 64) to two rounds (D = 256) per tile, rows past n come in as
    zero bytes."""
    pkv = require_gpu()
    from dataclasses import replace
    cfg = replace(W.PREFILL_CONFIGS[1], D=D, BS=BS, dtype="bf16", H=2, cache_dtype=cache)
    q_lens = [1, 31, 32, 33, 127, 128, 129, 0, 200, 5, 64]
    cached = [0, 0, 0, 0, 0, 1, 15, 9, 17, 300, 64]
    case = W.make_prefill_case(cfg, device="cuda", q_lens=q_lens, cached=cached, seed=79)
    print(f"prefill 8-bit boundaries {cache} D={D} BS={BS}", flush=True)
    k_pre, v_pre, gk, gv, gout = run_gpu(pkv, case)
    err = check(case, gk, gv, gout, oracle_run(case, k_pre, v_pre), f"{cache} D{D} BS{BS}")
    print(f"{cache} D={D} BS={BS}: max abs error {err:.3g}", flush=True)


def test_prefill_placement_invariance_is_bitwise():
    """Moving every physical block elsewhere (and renaming it in the tables)
    leaves the output bit for bit unchanged: the arithmetic follows logical
    positions only."""
    pkv = require_gpu()
    case = W.make_prefill_case(W.PREFILL_CONFIGS[4], device="cuda", S=16)
    _, _, gk, gv, out1 = run_gpu(pkv, case, keep_pre=False)
    perm = torch.randperm(case.NB, generator=torch.Generator().manual_seed(5)).to("cuda")
    k2 = torch.empty_like(gk)
    v2 = torch.empty_like(gv)
    k2[perm] = gk
    v2[perm] = gv
    tables2 = perm.to(torch.int32)[torch.from_numpy(case.block_tables).long().to("cuda")]
    out2 = torch.empty_like(out1)
    pkv.paged_attention_prefill(out2, case.q, k2, v2, tables2.contiguous(), torch.from_numpy(case.context_lens).cuda(),
                                torch.from_numpy(case.cu_q_lens).cuda(), case.max_q_len, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_prefill_shared_prefix_equals_duplicated_prefix():
    """Sequences mapping one shared physical prefix give bitwise the output
    they give with private copies of it."""
    pkv = require_gpu()
    case = W.make_prefill_case(W.PREFILL_CONFIGS[4], device="cuda", S=16)
    _, _, gk, gv, out1 = run_gpu(pkv, case, keep_pre=False)
    # give every sequence private copies of all its blocks
    BS = case.BS
    nb = [-(-int(n) // BS) for n in case.context_lens]
    total = sum(nb)
    k2 = torch.empty((total + 1,) + tuple(gk.shape[1:]), dtype=gk.dtype, device="cuda")
    v2 = torch.empty_like(k2)
    tables2 = np.zeros_like(case.block_tables)
    nxt = 0
    for s in range(case.S):
        src = torch.from_numpy(case.block_tables[s, :nb[s]].astype(np.int64)).cuda()
        k2[nxt:nxt + nb[s]] = gk[src]
        v2[nxt:nxt + nb[s]] = gv[src]
        tables2[s, :nb[s]] = np.arange(nxt, nxt + nb[s])
        tables2[s, nb[s]:] = total
        nxt += nb[s]
    k2[total] = float("nan")
    v2[total] = float("nan")
    out2 = torch.empty_like(out1)
    pkv.paged_attention_prefill(out2, case.q, k2, v2, torch.from_numpy(tables2).cuda(),
                                torch.from_numpy(case.context_lens).cuda(), torch.from_numpy(case.cu_q_lens).cuda(),
                                case.max_q_len, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_prefill_one_new_token_matches_the_decode_within_tolerance():
    """With one new token per sequence the prompt kernel computes the decode;
    both match the oracle's decode."""
    pkv = require_gpu()
    cfg = W.CONFIGS[2]
    case = W.make_case(cfg, device="cuda")
    dev = "cuda"
    pkv.reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache, torch.from_numpy(case.slot_mapping).to(dev))
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    cu = torch.arange(case.S + 1, dtype=torch.int32, device=dev)
    out_p = torch.empty_like(case.q)
    pkv.paged_attention_prefill(out_p, case.q, case.k_cache, case.v_cache, bt, cl, cu, 1, case.scale)
    out_d = torch.empty_like(case.q)
    pkv.paged_attention_decode(out_d, case.q, case.k_cache, case.v_cache, bt, cl, case.scale)
    torch.cuda.synchronize()
    want = oracle.paged_attention_decode(W.bits(case.q, "f16"), W.bits(case.k_cache, "f16"),
                                         W.bits(case.v_cache, "f16"), case.block_tables, case.context_lens,
                                         case.scale, "f16", "f16")
    assert np.abs(out_f64(out_d) - want).max() <= 2e-3
    # the prompt kernel's bound (module docstring); the softmax average of |V|
    # from the oracle run on V with its sign bits cleared
    avg_abs_v = oracle.paged_attention_decode(W.bits(case.q, "f16"), W.bits(case.k_cache, "f16"),
                                              abs_bits(W.bits(case.v_cache, "f16"), "f16"), case.block_tables,
                                              case.context_lens, case.scale, "f16", "f16")
    u = U_P["f16"]
    bound = 2e-3 + u * (avg_abs_v + np.abs(want)) / (1.0 - u) + OUT_REL["f16"] * np.abs(want)
    assert (np.abs(out_f64(out_p) - want) <= bound).all()


def test_prefill_rejects_unsupported_and_invalid():
    pkv = require_gpu()
    dev = "cuda"
    q = torch.zeros((4, 2, 128), dtype=torch.float32, device=dev)
    kc = torch.zeros((3, 2, 16, 128), dtype=torch.float32, device=dev)
    bt = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    cl = torch.full((1,), 4, dtype=torch.int32, device=dev)
    cu = torch.tensor([0, 4], dtype=torch.int32, device=dev)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attention_prefill(torch.empty_like(q), q, kc, kc, bt, cl, cu, 4, 0.1)
    assert e.value.status == pkv.PKV_ERR_UNSUPPORTED
    q16 = q.half()
    k16 = kc.half()
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attention_prefill(torch.empty_like(q16), q16, k16, k16, bt, cl, cu, 4, float("nan"))
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PagedKVError) as e:            # a 16-bit pool of the other format
        pkv.paged_attention_prefill(torch.empty_like(q16), q16, kc.bfloat16(), kc.bfloat16(), bt, cl, cu, 4, 0.1)
    assert e.value.status == pkv.PKV_ERR_UNSUPPORTED
    k8 = torch.zeros(kc.shape, dtype=torch.uint8, device=dev)
    for bad in (0.0, float("inf")):                       # 8-bit pools need finite positive scales
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_attention_prefill(torch.empty_like(q16), q16, k8, k8, bt, cl, cu, 4, 0.1, bad, 1.0)
        assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    # nothing to do
    pkv.paged_attention_prefill(torch.empty_like(q16), q16, k16, k16, bt, cl, cu, 0, 0.1)

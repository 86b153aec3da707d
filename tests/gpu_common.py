"""Helpers for the GPU parity tests: run one decode step through the C ABI
binding and the same step through the oracle, on the same seeded inputs.

The oracle's inputs are the generator's pre-step pools (never anything the
HIP path wrote): it applies its own block copies and cache write, then its
own decode.  Large pools are checked on a sample of sequences: only the
physical blocks those sequences (and their copy sources) touch are moved to
the host and renumbered 0..M-1, which the placement invariance pinned on the
CPU makes equivalent.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import pytest
import torch

import oracle
import workloads as W

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "e4m3": 3e-2, "i8": 3e-2}   # 8-bit KV formats alike
# largest relative rounding error of the output format (half an ulp)
OUT_REL = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# significant bits and smallest normal exponent of each output format
_PREC = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}
U32 = 2.0 ** -24                  # unit roundoff of fp32, the kernels' arithmetic

# The decode kernel's work split, as far as the error bound below needs it:
# partitions of 2048 tokens, 8 waves per workgroup, one 16-byte load per lane
# covering 16 / element-size head elements of a row.
PART_TOKENS = 2048
WAVES = 8


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_423_amd as pkv
    pkv.lib()          # raises if the library is missing: no fallback
    return pkv


def tol_for(case: W.Case) -> float:
    return TOL[case.cache_dtype]


@dataclass
class GpuStep:
    k_pre: torch.Tensor
    v_pre: torch.Tensor
    k_post: torch.Tensor
    v_post: torch.Tensor
    out: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor


def run_gpu_step(pkv, case: W.Case, keep_pre: bool = True, workspace=None) -> GpuStep:
    """copy_blocks (if any), reshape_and_cache, paged_attention_decode on the GPU."""
    dev = "cuda"
    c = case if case.k_cache.device.type == "cuda" else case.to(dev)
    k_pre = c.k_cache.clone() if keep_pre else None
    v_pre = c.v_cache.clone() if keep_pre else None
    kc, vc = c.k_cache, c.v_cache
    if case.copy_pairs.shape[0]:
        pkv.copy_blocks(kc, vc, torch.from_numpy(case.copy_pairs).to(dev))
    pkv.reshape_and_cache(c.key, c.value, kc, vc, torch.from_numpy(case.slot_mapping).to(dev),
                          case.k_scale, case.v_scale)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(c.q)
    pkv.paged_attention_decode(out, c.q, kc, vc, bt, cl, case.scale, case.k_scale, case.v_scale,
                               workspace=workspace)
    torch.cuda.synchronize()
    return GpuStep(k_pre, v_pre, kc, vc, out, bt, cl)


@dataclass
class OracleStep:
    seqs: List[int]
    blocks: np.ndarray           # physical ids of the mini pool, in mini order
    mapped: np.ndarray           # mini indices of the blocks the sampled sequences map
    k_post: np.ndarray           # oracle's mini pools after copy + write (bits)
    v_post: np.ndarray
    out: np.ndarray              # float64 [len(seqs), H, D]
    fp32_err: np.ndarray         # float64 [len(seqs), H]: bound on the kernel's fp32 arithmetic error


def oracle_step(case: W.Case, k_pre: torch.Tensor, v_pre: torch.Tensor,
                seqs: Optional[Sequence[int]] = None) -> OracleStep:
    """The same step in the oracle, restricted to ``seqs`` (all by default)."""
    seqs = list(range(case.S)) if seqs is None else list(seqs)
    BS, dt = case.BS, case.cache_dtype
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
    kb = W.bits(k_pre.index_select(0, idx), dt)
    vb = W.bits(v_pre.index_select(0, idx), dt)
    mini_pairs = np.array([(remap[a], remap[b]) for a, b in pairs], dtype=np.int64).reshape(-1, 2)
    kb, vb = oracle.copy_blocks(kb, vb, mini_pairs)
    sl = case.slot_mapping[seqs].astype(np.int64)
    mini_slots = np.array([remap[int(x) // BS] * BS + int(x) % BS for x in sl], dtype=np.int64)
    sel = torch.as_tensor(seqs, dtype=torch.long)
    key = W.bits(case.key.index_select(0, sel.to(case.key.device)), case.q_dtype)
    val = W.bits(case.value.index_select(0, sel.to(case.value.device)), case.q_dtype)
    kb, vb = oracle.reshape_and_cache(key, val, kb, vb, mini_slots, case.q_dtype, dt,
                                      case.k_scale, case.v_scale)
    tables = np.zeros((len(seqs), case.MB), dtype=np.int64)
    for i, s in enumerate(seqs):
        nb = -(-int(case.context_lens[s]) // BS)
        tables[i, :nb] = [remap[int(b)] for b in case.block_tables[s, :nb]]
    q = W.bits(case.q.index_select(0, sel.to(case.q.device)), case.q_dtype)
    out = oracle.paged_attention_decode(q, kb, vb, tables, case.context_lens[seqs], case.scale,
                                        case.q_dtype, dt, case.k_scale, case.v_scale)
    mapped = np.array([remap[b] for b in mapped_ids], dtype=np.int64)
    err = fp32_error_bound(case, q, kb, vb, tables, case.context_lens[seqs])
    return OracleStep(seqs, blocks, mapped, kb, vb, out, err)


def _head_scales(x, H):
    return np.broadcast_to(np.asarray(x, dtype=np.float64).reshape(-1), (H,)) if np.ndim(x) else np.full(H, float(x))


def fp32_error_bound(case: W.Case, q_bits, k_bits, v_bits, tables, lens) -> np.ndarray:
    """First-order bound on how far the decode kernel's fp32 result (before
    its rounding to the output format) can lie from the exact softmax
    average, per (sampled sequence, head).

    out = A / L with A = sum_t p_t V_t, L = sum_t p_t, p_t = 2^(z_t - m).
      * Accumulation: a term passes through at most G fp32 roundings on its
        way into A or L: 2R in its lane (R rows of the partition per lane,
        one FMA and one rescale each), 3 per shuffle level of the row-group
        merge (log2 of the rows per load), one per wave of the cross-wave
        merge, 3 per further partition in the merge kernel, 2 for the final
        division and scaling.  Factors that multiply A and L alike (the
        exponentials of the rescales and merges) cancel in A / L.  The
        result moves by at most 2^-24 G (sum p|V| + |out|) / L <= 2^-24 2G Vmax.
      * Weights: z_t = sum_d q'_d k_td is formed by EPL FMAs in a lane, then
        log2(LPR) cross-lane adds, with q' = q * scale * log2(e) rounded once:
        |dz| <= 2^-24 (EPL + log2 LPR + 1) Z, Z = max_t sum_d |q'_d k_td|.  A
        weight then carries relative error <= ln2 |dz| + 3 * 2^-24 (exp2 and the
        subtraction of m), which moves the output by at most twice that
        times Vmax.
    INT8 values enter the sums as byte + 128 (the offset comes off once per
    dot product and once per output), so their Vmax and Z use byte + 128.
    """
    S, H, D = q_bits.shape
    BS = case.BS
    cdt = case.cache_dtype
    eb = W.ELEM_BYTES[cdt]
    epl = 16 // eb                                  # elements per 16-byte load
    act = D // epl                                  # lanes holding part of a row
    lpr = 1 << max(0, math.ceil(math.log2(act)))    # lanes per row (power of two)
    rpl = 64 // lpr                                 # rows per wave-wide load
    ks = _head_scales(case.k_scale, H) if cdt in oracle.SCALED else np.ones(H)
    vs = _head_scales(case.v_scale, H) if cdt in oracle.SCALED else np.ones(H)
    qv = np.abs(oracle.decode(q_bits, case.q_dtype)) * (case.scale * 1.4426950408889634)
    err = np.zeros((S, H), dtype=np.float64)
    for i in range(S):
        n = int(lens[i])
        if n == 0:
            continue
        kr, vr, _ = oracle.gather_kv(k_bits, v_bits, tables[i:i + 1], np.array([n]))
        if cdt == "i8":
            kval = (kr.view(np.int8).astype(np.float64) + 128.0) * ks[None, :, None]
            vval = (vr.view(np.int8).astype(np.float64) + 128.0) * vs[None, :, None]
        else:
            kval = np.abs(oracle.decode(kr, cdt)) * ks[None, :, None]
            vval = np.abs(oracle.decode(vr, cdt)) * vs[None, :, None]
        vmax = vval.max(axis=(0, 2))                                   # [H]
        z = np.einsum("thd,hd->th", kval, qv[i]).max(axis=0)           # [H]
        parts = -(-n // PART_TOKENS)
        per_wave_blocks = -(-(-(-min(n, PART_TOKENS) // BS)) // WAVES)
        rows = per_wave_blocks * (BS // rpl)
        g = 2 * rows + 3 * int(math.log2(rpl)) + WAVES + 3 * (parts - 1) + 2
        eta = math.log(2.0) * (epl + math.log2(lpr) + 1) * U32 * z + 3 * U32
        err[i] = 2.0 * vmax * (U32 * g + eta)
    return err


def half_ulp(x: np.ndarray, fmt: str) -> np.ndarray:
    """Half the spacing of format ``fmt`` at magnitude x >= 0: the largest
    error of rounding a value of that magnitude to nearest."""
    p, emin = _PREC[fmt]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = f 2^e, f in [0.5, 1): binade 2^(e - 1)
    e = np.where(x == 0, emin + 1, e)        # zero and subnormals: the spacing of the smallest binade
    return np.ldexp(1.0, np.maximum(e - 1, emin) - p)


def decode_bound(case: W.Case, want: np.ndarray, fp32_err: np.ndarray) -> np.ndarray:
    """Per-element bound for a decode output against the exact result.

    The stated tolerance (1e-5 / 2e-3 / 3e-2) holds wherever the output
    format's own rounding leaves room for it: where half an ulp of the output
    at |want| is at most half the tolerance, the bound is the tolerance.
    Elsewhere (bf16 outputs of magnitude 0.5 or more, which short contexts
    give) no implementation that rounds to the format can promise the
    tolerance; the bound there is max(tol, half_ulp(|want| + c) + c), the
    rounding of a value that the fp32 arithmetic left within c of the exact
    one (c from fp32_error_bound)."""
    tol = tol_for(case)
    c = fp32_err[:, :, None]
    a = np.abs(want)
    rounding = half_ulp(a, case.q_dtype)
    allowed = np.maximum(tol, half_ulp(a + c, case.q_dtype) + c)
    return np.where(rounding <= tol / 2, tol, allowed)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_step(case: W.Case, g: GpuStep, o: OracleStep, label: str = "") -> float:
    """Bitwise pools on the blocks the sampled sequences map, attention within
    decode_bound (the stated tolerance wherever the output format's rounding
    leaves room for it); returns the max abs error."""
    idx = torch.from_numpy(o.blocks[o.mapped]).to(g.k_post.device)
    kg = W.bits(g.k_post.index_select(0, idx), case.cache_dtype)
    vg = W.bits(g.v_post.index_select(0, idx), case.cache_dtype)
    assert np.array_equal(kg, o.k_post[o.mapped]), f"{label}: K pool differs from the oracle"
    assert np.array_equal(vg, o.v_post[o.mapped]), f"{label}: V pool differs from the oracle"
    sel = torch.as_tensor(o.seqs, dtype=torch.long, device=g.out.device)
    got = out_f64(g.out.index_select(0, sel))
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    diff = np.abs(got - o.out)
    err = float(diff.max())
    bound = decode_bound(case, o.out, o.fp32_err)
    bad = diff > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(diff - bound)), diff.shape)
        raise AssertionError(f"{label}: {int(bad.sum())} elements over the bound; worst at seq {o.seqs[i[0]]} "
                             f"(n={int(case.context_lens[o.seqs[i[0]]])}) head {i[1]} dim {i[2]}: got {got[i]!r}, "
                             f"want {o.out[i]!r}, bound {bound[i]:.3g} (fp32 term {o.fp32_err[i[0], i[1]]:.3g})")
    return err


def assert_tolerance_budget(case: W.Case, o: OracleStep) -> None:
    """The full workloads: the output format's own rounding fits in the
    stated tolerance at every element, so the bound is the tolerance."""
    tol = tol_for(case)
    assert float(np.abs(o.out).max()) * OUT_REL[case.q_dtype] < tol
    assert (decode_bound(case, o.out, o.fp32_err) == tol).all()


def check_untouched(g: GpuStep, touched_blocks: Sequence[int]) -> None:
    """Blocks outside ``touched_blocks`` are bitwise unchanged by the step."""
    NB = g.k_pre.shape[0]
    mask = torch.ones(NB, dtype=torch.bool, device=g.k_pre.device)
    if len(touched_blocks):
        mask[torch.as_tensor(list(touched_blocks), device=g.k_pre.device)] = False
    for pre, post in ((g.k_pre, g.k_post), (g.v_pre, g.v_post)):
        a = pre[mask].view(torch.uint8) if pre.dtype != torch.uint8 else pre[mask]
        b = post[mask].view(torch.uint8) if post.dtype != torch.uint8 else post[mask]
        assert torch.equal(a, b), "a block outside the written slots and copy targets changed"


def touched(case: W.Case) -> List[int]:
    t = set(int(x) // case.BS for x in case.slot_mapping if x >= 0)
    t.update(int(b) for b in case.copy_pairs[:, 1])
    return sorted(t)


def sample_seqs(case: W.Case, k: int, seed: int = 0) -> List[int]:
    """Shortest, longest and k-2 more sequences (seeded)."""
    n = case.context_lens
    pick = {int(np.argmin(n)), int(np.argmax(n))}
    rng = np.random.default_rng(seed)
    for s in rng.permutation(case.S):
        if len(pick) >= min(k, case.S):
            break
        pick.add(int(s))
    return sorted(pick)

"""Pins for per-head scales of the 8-bit KV formats in the oracle (CPU).

An 8-bit pool (E4M3 or INT8) stores x / scale and holds byte * scale
("vLLM-v0.17.1技术解析：PagedAttention内存管理与显存优化技巧" §3.3 lists FP8 and
INT8 KV caches; the l189.com article on KV cache and PagedAttention §4 a
quantised cache in FP8 "and similar formats").  The scale may be one per
pool or one per head; with per-head scales, the rows of head h carry head h's
scale.  The oracle is checked against:

* brute force: pure-Python attention (decode and prompt) with each head's
  values decoded through struct / torch and multiplied by that head's own
  scale in a loop over heads;
* the library quantiser: torch's IEEE fp32 division by each head's scale,
  then its E4M3 cast (after the saturating clamp) or its half-to-even
  rounding and clamp to [-127, 127] for INT8, for the cache write;
* the special case: equal per-head scales give bitwise the per-pool form;
* a planted mistake: head 0's scale applied to every head must fail the
  brute-force pin and the quantiser pin;
* rejections: a scale list of the wrong length, or a non-positive scale.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import paged as opaged
from test_oracle_pins import brute_attention, build_paged, indep_values, random_bits, tiny_case
from test_oracle_prefill_pins import prefill_case

KS = np.array([0.011, 0.093, 0.047], dtype=np.float32).astype(np.float64)   # three heads, far apart
VS = np.array([0.071, 0.019, 0.1], dtype=np.float32).astype(np.float64)


def per_head_values(bits, fmt, scales):
    """[n, H, D] raw bits -> values, head h times scales[h], by explicit loops."""
    vals = indep_values(bits, fmt)
    out = np.empty_like(vals)
    for h in range(vals.shape[1]):
        out[:, h, :] = vals[:, h, :] * float(scales[h])
    return out


def brute_decode(q, qfmt, lk, lv, fmt, scale, ks, vs):
    S, H, D = q.shape
    qv = indep_values(q, qfmt)
    out = np.zeros((S, H, D))
    for s in range(S):
        K = per_head_values(lk[s], fmt, ks)
        V = per_head_values(lv[s], fmt, vs)
        for h in range(H):
            out[s, h] = brute_attention(list(qv[s, h]), K[:, h, :].tolist(), V[:, h, :].tolist(), scale)
    return out


def brute_prefill(q, qfmt, lk, lv, fmt, lens, cu, scale, ks, vs):
    Tq, H, D = q.shape
    qv = indep_values(q, qfmt)
    out = np.zeros((Tq, H, D))
    for s, n in enumerate(lens):
        n = int(n)
        K = per_head_values(lk[s], fmt, ks)
        V = per_head_values(lv[s], fmt, vs)
        qn = int(cu[s + 1] - cu[s])
        for i in range(qn):
            pos = n - qn + i
            for h in range(H):
                out[cu[s] + i, h] = brute_attention(list(qv[cu[s] + i, h]), K[: pos + 1, h, :].tolist(),
                                                    V[: pos + 1, h, :].tolist(), scale)
    return out


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("BS", [1, 4, 16])
def test_decode_with_head_scales_matches_brute_force(fmt, BS):
    rng = np.random.default_rng(300 + BS)
    q, qfmt, lk, lv, lens = tiny_case(rng, fmt, S=3, H=3, D=8)
    kc, vc, tables = build_paged(rng, lk, lv, BS, fmt)
    scale = 1 / math.sqrt(8)
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, scale, qfmt, fmt, KS, VS)
    want = brute_decode(q, qfmt, lk, lv, fmt, scale, KS, VS)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("BS", [1, 16])
def test_prefill_with_head_scales_matches_brute_force(fmt, BS):
    rng = np.random.default_rng(310 + BS)
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, fmt, [1, 9, 17, 30], [1, 9, 4, 12], H=3)
    kc, vc, tables = build_paged(rng, lk, lv, BS, fmt)
    scale = 0.3
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, scale, qfmt, fmt, KS, VS)
    want = brute_prefill(q, qfmt, lk, lv, fmt, lens, cu, scale, KS, VS)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _write_case(rng, src_fmt="f16"):
    H, D, BS, NB, T = 3, 16, 8, 6, 11
    x = rng.standard_normal((T, H, D)) * np.array([1.0, 8.0, 30.0])[None, :, None]
    x[0, 2, :4] = [np.inf, -np.inf, 60000, -60000]            # saturate, do not make NaN
    if src_fmt == "f16":
        bits = x.astype(np.float16).view(np.uint16)
        f32 = x.astype(np.float16).astype(np.float32)
    else:
        f32 = x.astype(np.float32)
        bits = (f32.view(np.uint32) >> 16).astype(np.uint16)   # bf16 bits (truncated input; exact value below)
        f32 = (bits.astype(np.uint32) << 16).view(np.float32)
    slots = rng.permutation(NB * BS)[:T].astype(np.int32)
    return H, D, BS, NB, bits, f32, slots


def _torch_quantise(f32, scales, fmt):
    x = torch.from_numpy(f32) / torch.from_numpy(scales.astype(np.float32))[None, :, None]   # IEEE fp32 division
    if fmt == "e4m3":
        return x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return torch.round(x).clamp(-127, 127).to(torch.int8).view(torch.uint8).numpy()             # half to even


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_cache_write_with_head_scales_matches_library_quantiser(fmt, src):
    rng = np.random.default_rng(320)
    H, D, BS, NB, bits, f32, slots = _write_case(rng, src)
    fill = 0x7F if fmt == "e4m3" else 0x80
    kc = np.full((NB, H, BS, D), fill, np.uint8)
    vc = kc.copy()
    k2, v2 = oracle.reshape_and_cache(bits, bits, kc, vc, slots, src, fmt, KS, VS)
    for pool, sc in ((k2, KS), (v2, VS)):
        ref = _torch_quantise(f32, sc, fmt)
        for i, s in enumerate(slots):
            assert (pool[s // BS, :, s % BS, :] == ref[i]).all()


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_equal_head_scales_are_the_per_pool_form(fmt):
    rng = np.random.default_rng(330)
    q, qfmt, lk, lv, lens = tiny_case(rng, fmt, S=3, H=3, D=8)
    kc, vc, tables = build_paged(rng, lk, lv, 4, fmt)
    ks, vs = float(np.float32(0.037)), float(np.float32(0.052))
    a = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.3, qfmt, fmt, ks, vs)
    b = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.3, qfmt, fmt, [ks] * 3, [vs] * 3)
    assert np.array_equal(a, b)
    q2, qfmt2, lk2, lv2, lens2, cu = prefill_case(rng, fmt, [5, 20], [5, 7], H=3)
    kc2, vc2, tables2 = build_paged(rng, lk2, lv2, 4, fmt)
    a = oracle.paged_attention_prefill(q2, kc2, vc2, tables2, lens2, cu, 0.3, qfmt2, fmt, ks, vs)
    b = oracle.paged_attention_prefill(q2, kc2, vc2, tables2, lens2, cu, 0.3, qfmt2, fmt, [ks] * 3, [vs] * 3)
    assert np.array_equal(a, b)
    H, D, BS, NB, bits, f32, slots = _write_case(rng)
    pool = np.zeros((NB, H, BS, D), np.uint8)
    a = oracle.reshape_and_cache(bits, bits, pool, pool, slots, "f16", fmt, ks, vs)
    b = oracle.reshape_and_cache(bits, bits, pool, pool, slots, "f16", fmt, [ks] * 3, [vs] * 3)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def _head0_everywhere(tensor_scale, H):
    s = np.asarray(tensor_scale, dtype=np.float64).reshape(-1)
    return np.full(H, float(s[0]))


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_head0_scale_for_every_head_fails_the_pins(fmt, monkeypatch):
    rng = np.random.default_rng(340)
    q, qfmt, lk, lv, lens = tiny_case(rng, fmt, S=3, H=3, D=8)
    kc, vc, tables = build_paged(rng, lk, lv, 4, fmt)
    want = brute_decode(q, qfmt, lk, lv, fmt, 0.3, KS, VS)
    H, D, BS, NB, bits, f32, slots = _write_case(rng)
    pool = np.zeros((NB, H, BS, D), np.uint8)
    ref = _torch_quantise(f32, KS, fmt)
    monkeypatch.setattr(opaged, "head_scales", _head0_everywhere)
    got = opaged.paged_attention_decode(q, kc, vc, tables, lens, 0.3, qfmt, fmt, KS, VS)
    assert not np.allclose(got, want, rtol=0, atol=1e-6)
    k2, _ = opaged.reshape_and_cache(bits, bits, pool, pool, slots, "f16", fmt, KS, VS)
    assert not all((k2[s // BS, :, s % BS, :] == ref[i]).all() for i, s in enumerate(slots))


def test_scale_lists_are_checked():
    rng = np.random.default_rng(350)
    q, qfmt, lk, lv, lens = tiny_case(rng, "e4m3", S=2, H=3, D=8)
    kc, vc, tables = build_paged(rng, lk, lv, 4, "e4m3")
    with pytest.raises(ValueError):
        oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.3, qfmt, "e4m3", [0.1, 0.2], 0.1)
    with pytest.raises(ValueError):
        oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.3, qfmt, "e4m3", 0.1, [0.1, 0.0, 0.2])
    assert np.array_equal(oracle.head_scales(0.25, 3), [0.25, 0.25, 0.25])

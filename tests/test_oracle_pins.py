"""Pins for the oracle's attention, cache write, block copy and gather (CPU).

The oracle is checked against things other than itself:

* brute force: a separately written contiguous attention (pure Python loops,
  math.exp) over the logical token rows, with values decoded by another
  route (struct / torch casts), on tiny inputs;
* a library special case: torch's scaled_dot_product_attention in float64;
* closed forms: one token, constant keys, constant values, one dominant key;
* the invariants the pages fix: the block mapping is invisible to the model
  ("在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战" §2.1), so any placement of
  physical blocks and any block size give the same gathered arrays and hence
  bitwise-equal float64 results; a prefix stored once and shared gives the
  same result as private copies (same page, §2.2);
* planted mistakes: mutants of the decode (swapped index, dropped scale,
  wrong operand, off-by-one length, wrong sign, wrong softmax axis) must each
  fail the brute-force pin, which shows that the pin has teeth.
"""

import math
import struct

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import paged as opaged

# ------------------------------------------------------------ independent helpers


def indep_values(bits, fmt):
    """Raw bits -> Python floats by a route that shares nothing with oracle.codecs."""
    flat = np.asarray(bits).reshape(-1)
    if fmt == "f32":
        vals = [struct.unpack("<f", struct.pack("<I", int(b)))[0] for b in flat]
    elif fmt == "f16":
        vals = [struct.unpack("<e", struct.pack("<H", int(b)))[0] for b in flat]
    elif fmt == "bf16":
        vals = [struct.unpack(">f", struct.pack(">HH", int(b), 0))[0] for b in flat]
    elif fmt == "e4m3":
        vals = torch.from_numpy(flat.astype(np.uint8)).view(torch.float8_e4m3fn).double().tolist()
    elif fmt == "i8":
        vals = [struct.unpack("<b", bytes([int(b)]))[0] for b in flat]
    else:
        raise ValueError(fmt)
    return np.array(vals, dtype=np.float64).reshape(np.shape(bits))


def brute_attention(q, K, V, scale):
    """softmax(scale * q . K^T) V for one head, pure Python; q [D], K/V [n][D]."""
    n, D = len(K), len(q)
    if n == 0:
        return [0.0] * D
    z = [scale * sum(q[d] * K[t][d] for d in range(D)) for t in range(n)]
    m = max(z)
    w = [math.exp(zt - m) for zt in z]
    tot = sum(w)
    return [sum(w[t] * V[t][d] for t in range(n)) / tot for d in range(D)]


def random_bits(rng, shape, fmt):
    x = rng.standard_normal(shape)
    if fmt == "f32":
        return x.astype(np.float32).view(np.uint32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if fmt == "bf16":
        return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine for inputs
    if fmt == "e4m3":
        return torch.from_numpy((x * 20).astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
    if fmt == "i8":
        return np.clip(np.rint(x * 30), -127, 127).astype(np.int8).view(np.uint8)
    raise ValueError(fmt)


NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F, "i8": 0x80}   # i8: -128, never stored


def build_paged(rng, logical_k, logical_v, BS, fmt, NB=None, order=None, tables_override=None):
    """Place per-sequence logical rows [n_s, H, D] into NaN-filled pools with a
    random placement; plain loops, no oracle code."""
    S = len(logical_k)
    H, D = logical_k[0].shape[1], logical_k[0].shape[2]
    nblk = [-(-lk.shape[0] // BS) for lk in logical_k]
    MB = max(1, max(nblk))
    NB = NB or (sum(nblk) + 3)
    order = list(rng.permutation(NB)) if order is None else list(order)
    dt = oracle.bits_dtype(fmt)
    kc = np.full((NB, H, BS, D), NAN_BITS[fmt], dtype=dt)
    vc = np.full((NB, H, BS, D), NAN_BITS[fmt], dtype=dt)
    tables = np.full((S, MB), order[-1], dtype=np.int32)   # padding -> a never-written block
    nxt = 0
    for s in range(S):
        for j in range(nblk[s]):
            tables[s, j] = order[nxt]
            nxt += 1
        for t in range(logical_k[s].shape[0]):
            b, o = tables[s, t // BS], t % BS
            for h in range(H):
                kc[b, h, o, :] = logical_k[s][t, h, :]
                vc[b, h, o, :] = logical_v[s][t, h, :]
    return kc, vc, tables


def tiny_case(rng, fmt, S=3, H=2, D=8, nmax=40, lens=None):
    lens = list(rng.integers(1, nmax + 1, size=S)) if lens is None else lens
    lk = [random_bits(rng, (n, H, D), fmt) for n in lens]
    lv = [random_bits(rng, (n, H, D), fmt) for n in lens]
    qfmt = "f16" if fmt in ("e4m3", "i8") else fmt
    q = random_bits(rng, (len(lens), H, D), qfmt)
    return q, qfmt, lk, lv, np.array(lens, dtype=np.int32)


def brute_case(q, qfmt, lk, lv, fmt, scale, k_scale=1.0, v_scale=1.0):
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    qv = indep_values(q, qfmt)
    for s in range(S):
        K = indep_values(lk[s], fmt) * (k_scale if fmt in ("e4m3", "i8") else 1.0)
        V = indep_values(lv[s], fmt) * (v_scale if fmt in ("e4m3", "i8") else 1.0)
        for h in range(H):
            out[s, h] = brute_attention(list(qv[s, h]), K[:, h, :].tolist(), V[:, h, :].tolist(), scale)
    return out


# ------------------------------------------------------------ brute force / library

@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "e4m3", "i8"])
@pytest.mark.parametrize("BS", [1, 4, 16])
def test_decode_matches_brute_force(fmt, BS):
    rng = np.random.default_rng(100 + BS)
    q, qfmt, lk, lv, lens = tiny_case(rng, fmt)
    kc, vc, tables = build_paged(rng, lk, lv, BS, fmt)
    ks, vs = (0.037, 0.052) if fmt in ("e4m3", "i8") else (1.0, 1.0)
    scale = 1 / math.sqrt(8)
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, scale, qfmt, fmt, ks, vs)
    want = brute_case(q, qfmt, lk, lv, fmt, scale, ks, vs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_decode_matches_torch_sdpa_float64():
    rng = np.random.default_rng(5)
    q, qfmt, lk, lv, lens = tiny_case(rng, "f32", S=3, H=2, D=8, nmax=40)
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    scale = 0.3
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, scale, "f32", "f32")
    for s in range(3):
        qs = torch.from_numpy(q[s].view(np.float32).astype(np.float64))[:, None, :]       # [H,1,D]
        K = torch.from_numpy(lk[s].view(np.float32).astype(np.float64)).transpose(0, 1)   # [H,n,D]
        V = torch.from_numpy(lv[s].view(np.float32).astype(np.float64)).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qs, K, V, scale=scale)[:, 0, :]
        np.testing.assert_allclose(got[s], ref.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ closed forms

def _one_seq(kc_rows, vc_rows, BS=4, fmt="f32"):
    rng = np.random.default_rng(0)
    return build_paged(rng, [kc_rows], [vc_rows], BS, fmt)


def test_single_token_returns_v0_exactly():
    rng = np.random.default_rng(11)
    for fmt in ("f32", "f16", "bf16"):
        q, qfmt, lk, lv, lens = tiny_case(rng, fmt, S=2, H=2, D=8, lens=[1, 1])
        kc, vc, tables = build_paged(rng, lk, lv, 16, fmt)
        got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.5, qfmt, fmt)
        for s in range(2):
            assert (got[s] == oracle.decode(lv[s][0], fmt)).all()


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(12)
    q, qfmt, lk, lv, lens = tiny_case(rng, "f32", S=2, H=2, D=8, lens=[37, 5])
    q[:] = 0
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.5, "f32", "f32")
    for s in range(2):
        mean = lv[s].view(np.float32).astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(got[s], mean, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_and_constant_values_give_the_row():
    rng = np.random.default_rng(13)
    q, qfmt, lk, lv, lens = tiny_case(rng, "f32", S=1, H=2, D=8, lens=[23])
    lk[0][:] = lk[0][0]
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.5, "f32", "f32")
    np.testing.assert_allclose(got[0], lv[0].view(np.float32).astype(np.float64).mean(axis=0), atol=1e-14)
    lk2 = [random_bits(rng, (23, 2, 8), "f32")]
    lv2 = [np.broadcast_to(lv[0][4], (23, 2, 8)).copy()]
    kc, vc, tables = build_paged(rng, lk2, lv2, 4, "f32")
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.5, "f32", "f32")
    np.testing.assert_allclose(got[0], lv[0][4].view(np.float32).astype(np.float64), atol=1e-14)


def test_one_dominant_key_selects_its_value():
    D, n, j = 8, 30, 17
    K = np.zeros((n, 1, D), np.float32)
    K[:, 0, 1] = 1.0
    K[j, 0, 0] = 10.0
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 10.0
    rng = np.random.default_rng(14)
    V = rng.standard_normal((n, 1, D)).astype(np.float32)
    kc, vc, tables = build_paged(rng, [K.view(np.uint32)], [V.view(np.uint32)], 4, "f32")
    got = oracle.paged_attention_decode(q.view(np.uint32), kc, vc, tables, [n], 10.0, "f32", "f32")
    assert (got[0, 0] == V[j, 0].astype(np.float64)).all()     # exp(-1000) underflows to 0


def test_empty_context_gives_zeros():
    rng = np.random.default_rng(15)
    q, qfmt, lk, lv, lens = tiny_case(rng, "f16", S=2, H=2, D=8, lens=[3, 5])
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f16")
    got = oracle.paged_attention_decode(q, kc, vc, tables, [0, 5], 0.5, "f16", "f16")
    assert (got[0] == 0).all() and np.isfinite(got[1]).all()


def test_padding_is_never_read():
    # tables are padded with a NaN block and partial last blocks are NaN-filled
    rng = np.random.default_rng(16)
    q, qfmt, lk, lv, lens = tiny_case(rng, "bf16", S=3, H=2, D=8, lens=[1, 17, 31])
    kc, vc, tables = build_paged(rng, lk, lv, 16, "bf16")
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.5, "bf16", "bf16")
    assert np.isfinite(got).all()


def test_decode_rejects_bad_indices():
    rng = np.random.default_rng(17)
    q, qfmt, lk, lv, lens = tiny_case(rng, "f32", S=1, H=1, D=8, lens=[5])
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    bad = tables.copy()
    bad[0, 0] = kc.shape[0]
    with pytest.raises(ValueError):
        oracle.paged_attention_decode(q, kc, vc, bad, lens, 0.5, "f32", "f32")
    with pytest.raises(ValueError):
        oracle.paged_attention_decode(q, kc, vc, tables, [tables.shape[1] * 4 + 1], 0.5, "f32", "f32")


# ------------------------------------------------------------ invariants

@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), BS=st.sampled_from([1, 2, 4, 8, 16, 32]),
       BS2=st.sampled_from([1, 2, 4, 8, 16, 32]), fmt=st.sampled_from(["f32", "f16", "bf16", "e4m3"]))
def test_placement_and_block_size_invariance(seed, BS, BS2, fmt):
    rng = np.random.default_rng(seed)
    q, qfmt, lk, lv, lens = tiny_case(rng, fmt, S=3, H=2, D=8, nmax=40)
    a = build_paged(rng, lk, lv, BS, fmt)
    b = build_paged(rng, lk, lv, BS, fmt, NB=a[0].shape[0] + 5)      # another placement, bigger pool
    c = build_paged(rng, lk, lv, BS2, fmt)                           # another block size
    outs = [oracle.paged_attention_decode(q, kc, vc, t, lens, 0.35, qfmt, fmt, 0.05, 0.07)
            for kc, vc, t in (a, b, c)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_prefix_equals_duplicated():
    rng = np.random.default_rng(18)
    BS, H, D, P = 4, 2, 8, 12          # a 12-token prefix = 3 full blocks
    prefix_k = random_bits(rng, (P, H, D), "f16")
    prefix_v = random_bits(rng, (P, H, D), "f16")
    tails = [5, 0, 9]
    lk = [np.concatenate([prefix_k, random_bits(rng, (n, H, D), "f16")]) for n in tails]
    lv = [np.concatenate([prefix_v, random_bits(rng, (n, H, D), "f16")]) for n in tails]
    lens = np.array([P + n for n in tails], np.int32)
    q = random_bits(rng, (3, H, D), "f16")
    kc, vc, dup_tables = build_paged(rng, lk, lv, BS, "f16")
    dup = oracle.paged_attention_decode(q, kc, vc, dup_tables, lens, 0.4, "f16", "f16")
    # shared: point every sequence's first three logical blocks at sequence 0's blocks
    shared_tables = dup_tables.copy()
    shared_tables[1:, :3] = dup_tables[0, :3]
    shared = oracle.paged_attention_decode(q, kc, vc, shared_tables, lens, 0.4, "f16", "f16")
    assert np.array_equal(dup, shared)


# ------------------------------------------------------------ planted mistakes

def _mutant(kind):
    def decode_seq(q_bits_s, k_cache_bits, v_cache_bits, row, n, scale, q_dtype, cache_dtype,
                   k_scale=1.0, v_scale=1.0):
        H, D = q_bits_s.shape
        BS = k_cache_bits.shape[2]
        t = np.arange(n - 1 if kind == "short" else n)
        logical, off = (t % BS, t // BS) if kind == "swap_index" else (t // BS, t % BS)
        phys = np.asarray(row)[np.minimum(logical, len(row) - 1)]
        off = np.minimum(off, BS - 1)
        q = oracle.decode(q_bits_s, q_dtype)
        K = oracle.decode(k_cache_bits[phys, :, off, :], cache_dtype)
        V = oracle.decode((k_cache_bits if kind == "v_is_k" else v_cache_bits)[phys, :, off, :], cache_dtype)
        sc = 1.0 if kind == "no_scale" else (-scale if kind == "sign" else scale)
        z = sc * np.einsum("thd,hd->ht", K, q)
        ax = 0 if kind == "axis" else 1
        w = np.exp(z - z.max(axis=ax, keepdims=True))
        p = w / w.sum(axis=ax, keepdims=True)
        return np.einsum("ht,thd->hd", p, V)
    return decode_seq


@pytest.mark.parametrize("kind", ["swap_index", "short", "v_is_k", "no_scale", "sign", "axis"])
def test_planted_mistakes_fail_the_brute_force_pin(kind, monkeypatch):
    rng = np.random.default_rng(19)
    q, qfmt, lk, lv, lens = tiny_case(rng, "f32", S=3, H=2, D=8, lens=[37, 22, 9])
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    want = brute_case(q, qfmt, lk, lv, "f32", 0.5)
    monkeypatch.setattr(opaged, "paged_attention_decode_seq", _mutant(kind))
    with np.errstate(all="ignore"):
        got = opaged.paged_attention_decode(q, kc, vc, tables, lens, 0.5, "f32", "f32")
    assert not np.allclose(got, want, rtol=0, atol=1e-6, equal_nan=False)


# ------------------------------------------------------------ cache write / copy / gather

def test_reshape_and_cache_places_rows_and_leaves_the_rest(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "slot_mapping_example.json")))
    BS = g["block_size"]
    rng = np.random.default_rng(20)
    H, D, NB = 2, 8, 10
    kc = random_bits(rng, (NB, H, BS, D), "f16")
    vc = random_bits(rng, (NB, H, BS, D), "f16")
    slots = np.array([e["slot"] for e in g["expect_slots"]], np.int32)
    T = slots.size
    key = random_bits(rng, (T, H, D), "f16")
    val = random_bits(rng, (T, H, D), "f16")
    slots_with_pad = np.concatenate([slots, [-1]]).astype(np.int32)
    key_p = np.concatenate([key, random_bits(rng, (1, H, D), "f16")])
    val_p = np.concatenate([val, random_bits(rng, (1, H, D), "f16")])
    k2, v2 = oracle.reshape_and_cache(key_p, val_p, kc, vc, slots_with_pad, "f16", "f16")
    touched = np.zeros((NB, BS), bool)
    for i, e in enumerate(g["expect_slots"]):
        blk = g["tables"][e["seq"]][e["token"] // BS]
        off = e["token"] % BS
        assert e["slot"] == blk * BS + off
        assert (k2[blk, :, off, :] == key[i]).all() and (v2[blk, :, off, :] == val[i]).all()
        touched[blk, off] = True
    assert (k2.transpose(0, 2, 1, 3)[~touched] == kc.transpose(0, 2, 1, 3)[~touched]).all()
    assert (v2.transpose(0, 2, 1, 3)[~touched] == vc.transpose(0, 2, 1, 3)[~touched]).all()
    assert np.dtype(np.int32).itemsize == g["slot_mapping_bytes_per_token"]


def test_reshape_and_cache_fp8_matches_library_quantiser():
    rng = np.random.default_rng(21)
    H, D, BS, NB, T = 3, 16, 8, 6, 11
    key = (rng.standard_normal((T, H, D)) * 30).astype(np.float16)
    key[0, 0, :4] = [np.inf, -np.inf, 60000, -60000]          # saturate, do not make NaN
    val = (rng.standard_normal((T, H, D)) * 0.01).astype(np.float16)
    kc = np.full((NB, H, BS, D), 0x7F, np.uint8)
    vc = np.full((NB, H, BS, D), 0x7F, np.uint8)
    slots = rng.permutation(NB * BS)[:T].astype(np.int32)
    ks, vs = float(np.float32(0.0625)), float(np.float32(0.0123))
    k2, v2 = oracle.reshape_and_cache(key.view(np.uint16), val.view(np.uint16), kc, vc, slots,
                                      "f16", "e4m3", ks, vs)
    for src, pool, sc in ((key, k2, ks), (val, v2, vs)):
        x = torch.from_numpy(src.astype(np.float32)) / torch.tensor(sc, dtype=torch.float32)
        ref = x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        for i, s in enumerate(slots):
            assert (pool[s // BS, :, s % BS, :] == ref[i]).all()
    assert k2[slots[0] // BS, 0, slots[0] % BS, 0] == 0x7E and k2[slots[0] // BS, 0, slots[0] % BS, 1] == 0xFE


def test_reshape_and_cache_rejects_duplicate_slots():
    kc = np.zeros((2, 1, 4, 8), np.uint32)
    key = np.zeros((2, 1, 8), np.uint32)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(key, key, kc, kc, np.array([3, 3], np.int32), "f32", "f32")
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(key, key, kc, kc, np.array([3, 8], np.int32), "f32", "f32")


def test_copy_blocks_semantics():
    rng = np.random.default_rng(22)
    kc = random_bits(rng, (8, 2, 4, 8), "bf16")
    vc = random_bits(rng, (8, 2, 4, 8), "bf16")
    pairs = np.array([[1, 5], [1, 6], [3, 0]], np.int32)
    k2, v2 = oracle.copy_blocks(kc, vc, pairs)
    for s, d in pairs:
        assert (k2[d] == kc[s]).all() and (v2[d] == vc[s]).all()
    for b in (1, 2, 3, 4, 7):
        assert (k2[b] == kc[b]).all() and (v2[b] == vc[b]).all()
    k3, v3 = oracle.copy_blocks(kc, vc, pairs[::-1])
    assert (k3 == k2).all() and (v3 == v2).all()
    for bad in ([[1, 5], [2, 5]], [[1, 5], [5, 6]], [[1, 8]]):
        with pytest.raises(ValueError):
            oracle.copy_blocks(kc, vc, np.array(bad, np.int32))


def test_gather_matches_loops():
    rng = np.random.default_rng(23)
    q, qfmt, lk, lv, lens = tiny_case(rng, "e4m3", S=3, H=2, D=8, nmax=40)
    kc, vc, tables = build_paged(rng, lk, lv, 8, "e4m3")
    ko, vo, cu = oracle.gather_kv(kc, vc, tables, lens)
    assert list(cu) == [0] + list(np.cumsum(lens))
    for s in range(3):
        assert (ko[cu[s]:cu[s + 1]] == lk[s]).all() and (vo[cu[s]:cu[s + 1]] == lv[s]).all()


def test_block_bytes_match_the_pages(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "sizes.json")))
    b = g["block_bytes"]
    # one [H, BS, D] tile in each of the K and V pools
    tile = np.zeros((b["num_heads"], b["block_size"], b["head_size"]), np.uint32)
    assert 2 * tile.nbytes == b["bytes"]
    t = g["kv_bytes_per_token_per_layer"]
    assert 2 * t["hidden"] * t["elem_bytes"] == t["bytes"]
    assert t["bytes"] * t["layers"] == t["bytes_all_layers"]

"""Pins for the oracle's multi-query (prompt) paged attention (CPU).

New token i of a sequence that holds n tokens, q of them new, sits at
position n - q + i and attends to positions 0 .. n - q + i ("在A10G上榨干
LLaMA-7B：vLLM与PagedAttention实战" §2.1 step 1 and §2.2: a prompt's K/V are
stored in its blocks and then used, and a shared prompt prefix is stored
once).  The oracle is checked against:

* brute force: pure-Python loops per query over the visible positions, with
  values decoded through struct / torch casts;
* a library special case: torch's scaled_dot_product_attention in float64,
  with is_causal for whole prompts and an explicit bottom-right-aligned mask
  when a cached prefix precedes the new tokens;
* closed forms: the first token of a prompt sees only itself (out = v_0);
  identical keys give the running mean of V;
* the decode as the one-new-token case;
* invariants: physical placement and block size (bitwise), and chunking a
  prompt (the second chunk's rows equal the whole prompt's rows);
* planted mistakes: a top-left-aligned mask, a strict mask, an off-by-one
  position and a mask ignoring the cached prefix must each fail brute force.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import paged as opaged
from test_oracle_pins import brute_attention, build_paged, indep_values, random_bits


def prefill_case(rng, fmt, lens, qlens, H=2, D=8):
    """Per-sequence logical rows, packed new-token queries and cu_q_lens."""
    lk = [random_bits(rng, (n, H, D), fmt) for n in lens]
    lv = [random_bits(rng, (n, H, D), fmt) for n in lens]
    qfmt = "f16" if fmt in ("e4m3", "i8") else fmt
    q = random_bits(rng, (int(sum(qlens)), H, D), qfmt)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(qlens)
    return q, qfmt, lk, lv, np.array(lens, dtype=np.int32), cu


def brute_prefill(q, qfmt, lk, lv, fmt, lens, cu, scale, k_scale=1.0, v_scale=1.0):
    Tq, H, D = q.shape
    out = np.zeros((Tq, H, D))
    qv = indep_values(q, qfmt)
    for s, n in enumerate(lens):
        n = int(n)
        K = indep_values(lk[s], fmt) * (k_scale if fmt in ("e4m3", "i8") else 1.0)
        V = indep_values(lv[s], fmt) * (v_scale if fmt in ("e4m3", "i8") else 1.0)
        qn = int(cu[s + 1] - cu[s])
        for i in range(qn):
            pos = n - qn + i
            for h in range(H):
                out[cu[s] + i, h] = brute_attention(list(qv[cu[s] + i, h]), K[: pos + 1, h, :].tolist(),
                                                    V[: pos + 1, h, :].tolist(), scale)
    return out


LENS = [1, 7, 16, 17, 40, 33]
QLENS = [1, 7, 16, 5, 40, 1]          # whole prompts, part prompts after a cached prefix, decode rows


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "e4m3", "i8"])
@pytest.mark.parametrize("BS", [1, 4, 16])
def test_prefill_matches_brute_force(fmt, BS):
    rng = np.random.default_rng(200 + BS)
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, fmt, LENS, QLENS)
    kc, vc, tables = build_paged(rng, lk, lv, BS, fmt)
    ks, vs = (0.041, 0.066) if fmt in ("e4m3", "i8") else (1.0, 1.0)
    scale = 1 / math.sqrt(8)
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, scale, qfmt, fmt, ks, vs)
    want = brute_prefill(q, qfmt, lk, lv, fmt, lens, cu, scale, ks, vs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_prefill_matches_torch_sdpa_float64():
    rng = np.random.default_rng(7)
    lens, qlens = [64, 50, 50, 23], [64, 50, 18, 1]
    H, D = 3, 16
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "f32", lens, qlens, H=H, D=D)
    kc, vc, tables = build_paged(rng, lk, lv, 16, "f32")
    scale = 0.3
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, scale, "f32", "f32")
    qv = torch.from_numpy(indep_values(q, "f32"))
    for s, n in enumerate(lens):
        n, qn = int(n), int(cu[s + 1] - cu[s])
        Q = qv[cu[s]:cu[s + 1]].permute(1, 0, 2)                           # [H, q, D]
        K = torch.from_numpy(indep_values(lk[s], "f32")).permute(1, 0, 2)  # [H, n, D]
        V = torch.from_numpy(indep_values(lv[s], "f32")).permute(1, 0, 2)
        if qn == n:
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
        else:
            mask = torch.ones(qn, n, dtype=torch.bool).tril(diagonal=n - qn)   # bottom-right aligned
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_prefill_first_token_sees_only_itself():
    rng = np.random.default_rng(8)
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "bf16", [30, 9], [30, 9])
    kc, vc, tables = build_paged(rng, lk, lv, 4, "bf16")
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, 0.5, "bf16", "bf16")
    for s in range(2):
        assert np.array_equal(got[cu[s]], indep_values(lv[s][0], "bf16"))


def test_prefill_identical_keys_give_running_mean():
    rng = np.random.default_rng(9)
    n, H, D = 20, 2, 8
    lk = [np.repeat(random_bits(rng, (1, H, D), "f32"), n, axis=0)]
    lv = [random_bits(rng, (n, H, D), "f32")]
    q = random_bits(rng, (n, H, D), "f32")
    cu = np.array([0, n])
    kc, vc, tables = build_paged(rng, lk, lv, 16, "f32")
    got = oracle.paged_attention_prefill(q, kc, vc, tables, np.array([n]), cu, 0.7, "f32", "f32")
    V = indep_values(lv[0], "f32")
    want = np.cumsum(V, axis=0) / np.arange(1, n + 1)[:, None, None]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_prefill_with_one_new_token_is_the_decode():
    rng = np.random.default_rng(10)
    lens = [5, 16, 33, 1]
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "f16", lens, [1, 1, 1, 1])
    kc, vc, tables = build_paged(rng, lk, lv, 16, "f16")
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, 0.35, "f16", "f16")
    dec = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.35, "f16", "f16")
    np.testing.assert_allclose(got, dec, rtol=0, atol=1e-13)


@pytest.mark.parametrize("BS", [1, 2, 8, 32])
def test_prefill_placement_and_block_size_invariance(BS):
    rng = np.random.default_rng(11)
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "f16", LENS, QLENS)
    kc, vc, tables = build_paged(np.random.default_rng(1), lk, lv, 16, "f16")
    base = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, 0.4, "f16", "f16")
    kc2, vc2, tables2 = build_paged(np.random.default_rng(BS), lk, lv, BS, "f16")
    other = oracle.paged_attention_prefill(q, kc2, vc2, tables2, lens, cu, 0.4, "f16", "f16")
    assert np.array_equal(base, other)


def test_prefill_chunking_matches_whole_prompt():
    """A prompt done in two chunks (the second one after the first is cached)
    gives the whole prompt's rows for the second chunk."""
    rng = np.random.default_rng(12)
    n, split = 45, 19
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "bf16", [n], [n])
    kc, vc, tables = build_paged(rng, lk, lv, 16, "bf16")
    whole = oracle.paged_attention_prefill(q, kc, vc, tables, lens, cu, 0.4, "bf16", "bf16")
    second = oracle.paged_attention_prefill(q[split:], kc, vc, tables, lens, np.array([0, n - split]), 0.4,
                                            "bf16", "bf16")
    np.testing.assert_allclose(second, whole[split:], rtol=0, atol=1e-13)
    # and the first chunk, run while only its own tokens are cached
    first = oracle.paged_attention_prefill(q[:split], kc, vc, tables, np.array([split]), np.array([0, split]),
                                           0.4, "bf16", "bf16")
    np.testing.assert_allclose(first, whole[:split], rtol=0, atol=1e-13)


def test_prefill_rejects_more_new_tokens_than_cached():
    rng = np.random.default_rng(13)
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "f32", [4], [4])
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    with pytest.raises(ValueError):
        oracle.paged_attention_prefill(q, kc, vc, tables, np.array([3]), cu, 1.0, "f32", "f32")


# ------------------------------------------------------------ planted mistakes

def _mutant(kind):
    def seq(q_bits_s, k_cache_bits, v_cache_bits, row, n, scale, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0):
        qn, H, D = q_bits_s.shape
        BS = k_cache_bits.shape[2]
        qv = oracle.decode(q_bits_s, q_dtype)
        K = opaged._cache_value(opaged.gather_seq_rows(k_cache_bits, row, n, BS), cache_dtype, k_scale)
        V = opaged._cache_value(opaged.gather_seq_rows(v_cache_bits, row, n, BS), cache_dtype, v_scale)
        i = np.arange(qn)
        pos = {"top_left": i, "off_by_one": n - qn + i + 1, "strict": n - qn + i, "no_prefix": n - qn + i}[kind]
        t = np.arange(n)[None, :]
        visible = {"top_left": t <= pos[:, None], "off_by_one": t <= pos[:, None],
                   "strict": (t < pos[:, None]) | (t == 0),
                   "no_prefix": (t <= pos[:, None]) & (t >= n - qn)}[kind]
        out = np.empty((qn, H, D))
        for h in range(H):
            z = np.where(visible, scale * (qv[:, h] @ K[:, h].T), -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            out[:, h] = (w / w.sum(axis=1, keepdims=True)) @ V[:, h]
        return out
    return seq


@pytest.mark.parametrize("kind", ["top_left", "off_by_one", "strict", "no_prefix"])
def test_planted_mask_mistakes_fail_brute_force(kind, monkeypatch):
    rng = np.random.default_rng(14)
    q, qfmt, lk, lv, lens, cu = prefill_case(rng, "f32", [20, 17], [8, 17])
    kc, vc, tables = build_paged(rng, lk, lv, 4, "f32")
    want = brute_prefill(q, qfmt, lk, lv, "f32", lens, cu, 0.5)
    monkeypatch.setattr(opaged, "paged_attention_prefill_seq", _mutant(kind))
    got = opaged.paged_attention_prefill(q, kc, vc, tables, lens, cu, 0.5, "f32", "f32")
    assert not np.allclose(got, want, rtol=0, atol=1e-6)

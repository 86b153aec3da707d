"""Pins for the oracle's block swap between two pools (CPU).

Swapping moves whole blocks between the GPU pools and a host swap space
("vLLM-v0.17.1技术解析" §4.1; "在A10G上榨干LLaMA-7B" §5.2).  Checked here: a
round trip out and back in restores the blocks bit for bit; blocks not
named are untouched; a block brought back to a different place, with the
table renamed to match, gives the same decode (the block mapping is
invisible to the model, "在A10G上榨干LLaMA-7B" §2.1); invalid pair lists are
rejected; a planted mistake (swapping K with V) is caught.
"""

import numpy as np
import pytest

import oracle
from oracle import paged as opaged
from test_oracle_pins import build_paged, random_bits


def _pools(rng, NB, H=2, BS=4, D=8, fmt="f16"):
    return random_bits(rng, (NB, H, BS, D), fmt), random_bits(rng, (NB, H, BS, D), fmt)


def test_round_trip_restores_blocks_and_leaves_the_rest():
    rng = np.random.default_rng(1)
    gk, gv = _pools(rng, 12)
    hk, hv = _pools(rng, 5)
    out_pairs = np.array([[3, 0], [7, 4], [11, 2]])
    hk2, hv2 = oracle.swap_blocks(gk, gv, hk, hv, out_pairs)
    for s, d in out_pairs:
        assert np.array_equal(hk2[d], gk[s]) and np.array_equal(hv2[d], gv[s])
    for d in (1, 3):
        assert np.array_equal(hk2[d], hk[d]) and np.array_equal(hv2[d], hv[d])
    # clobber the GPU blocks, then bring them back to other places
    gk_c, gv_c = gk.copy(), gv.copy()
    gk_c[[3, 7, 11]] = 0
    gv_c[[3, 7, 11]] = 0
    in_pairs = np.array([[0, 5], [4, 9], [2, 1]])
    gk3, gv3 = oracle.swap_blocks(hk2, hv2, gk_c, gv_c, in_pairs)
    assert np.array_equal(gk3[5], gk[3]) and np.array_equal(gk3[9], gk[7]) and np.array_equal(gk3[1], gk[11])
    assert np.array_equal(gv3[5], gv[3]) and np.array_equal(gv3[9], gv[7]) and np.array_equal(gv3[1], gv[11])


def test_swapped_in_elsewhere_gives_the_same_decode():
    rng = np.random.default_rng(2)
    lens = [9, 14]
    H, D, BS = 2, 8, 4
    lk = [random_bits(rng, (n, H, D), "f16") for n in lens]
    lv = [random_bits(rng, (n, H, D), "f16") for n in lens]
    q = random_bits(rng, (2, H, D), "f16")
    kc, vc, tables = build_paged(rng, lk, lv, BS, "f16", NB=12)
    want = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.4, "f16", "f16")
    # swap sequence 1's blocks out, reuse the GPU blocks, swap back to fresh ids
    used = [int(b) for b in tables[1, : -(-lens[1] // BS)]]
    host_k = np.zeros((len(used),) + kc.shape[1:], dtype=kc.dtype)
    host_v = np.zeros_like(host_k)
    host_k, host_v = oracle.swap_blocks(kc, vc, host_k, host_v, [[b, i] for i, b in enumerate(used)])
    busy = set(int(b) for b in tables[0, : -(-lens[0] // BS)]) | set(used)
    fresh = [b for b in range(kc.shape[0]) if b not in busy][: len(used)]
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[used] = 0x7E00
    vc2[used] = 0x7E00
    kc2, vc2 = oracle.swap_blocks(host_k, host_v, kc2, vc2, [[i, b] for i, b in enumerate(fresh)])
    tables2 = tables.copy()
    tables2[1, : len(fresh)] = fresh
    got = oracle.paged_attention_decode(q, kc2, vc2, tables2, lens, 0.4, "f16", "f16")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("pairs", [[[0, 1], [2, 1]], [[-1, 0]], [[0, 9]], [[12, 0]]])
def test_invalid_pairs_rejected(pairs):
    rng = np.random.default_rng(3)
    gk, gv = _pools(rng, 12)
    hk, hv = _pools(rng, 5)
    with pytest.raises(ValueError):
        oracle.swap_blocks(gk, gv, hk, hv, pairs)


def test_mismatched_block_shapes_rejected():
    rng = np.random.default_rng(4)
    gk, gv = _pools(rng, 12, BS=4)
    hk, hv = _pools(rng, 5, BS=8)
    with pytest.raises(ValueError):
        oracle.swap_blocks(gk, gv, hk, hv, [[0, 0]])


def test_planted_k_v_mixup_is_caught(monkeypatch):
    rng = np.random.default_rng(5)
    gk, gv = _pools(rng, 6)
    hk, hv = _pools(rng, 3)
    good_k, good_v = oracle.swap_blocks(gk, gv, hk, hv, [[1, 0]])

    def mutant(src_k, src_v, dst_k, dst_v, pairs):
        k, v = dst_k.copy(), dst_v.copy()
        for s, d in np.asarray(pairs).reshape(-1, 2):
            k[d], v[d] = src_v[s], src_k[s]
        return k, v
    monkeypatch.setattr(opaged, "swap_blocks", mutant)
    bad_k, bad_v = opaged.swap_blocks(gk, gv, hk, hv, [[1, 0]])
    assert not (np.array_equal(bad_k, good_k) and np.array_equal(bad_v, good_v))
    # the round-trip check above would fail for it
    assert not np.array_equal(bad_k[0], gk[1])

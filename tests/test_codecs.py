"""Pins for the oracle's number codecs (CPU only).

Every decoder is checked against an independent route to the same value:
the OCP E4M3 table printed in the specification (tests/golden/e4m3_values.json),
torch's CPU float8/bfloat16/float16 casts, and Python's struct module.  The
encoder is checked at every rounding midpoint, at saturation, NaN and in the
subnormal range, and against torch's CPU cast after clamping (clamping makes
torch's own overflow rule irrelevant).
"""

import json
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import codecs

pytestmark = []


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- e4m3 decode

def test_e4m3_decode_spec_values(golden_dir):
    g = _golden(golden_dir, "e4m3_values.json")
    for row in g["codes"]:
        b = int(row["byte"], 16)
        got = float(codecs.e4m3_decode(np.array([b], np.uint8))[0])
        if row["value"] == "nan":
            assert math.isnan(got), row
        else:
            assert got == row["value"], row
            assert math.copysign(1.0, got) == math.copysign(1.0, row["value"]), row


def test_e4m3_decode_all_256_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (ours[~nan] == ref[~nan]).all()
    assert (np.signbit(ours[~nan]) == np.signbit(ref[~nan])).all()


def test_e4m3_value_set_properties():
    v = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(v) > 0).all()                    # codes 0..126 increase strictly
    assert v[-1] == 448.0 and v[1] == 2.0 ** -9 and v[8] == 2.0 ** -6
    assert (np.diff(v[:9]) == 2.0 ** -9).all()       # subnormal spacing continues into the first binade


# ---------------------------------------------------------------- e4m3 encode

def test_e4m3_encode_exact_values_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes)
    assert (codecs.e4m3_encode(vals) == codes).all()


def test_e4m3_encode_midpoints_tie_to_even():
    pos = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2                                # exact in float64
    codes = codecs.e4m3_encode(mid)
    lo_code = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lo_code % 2 == 0, lo_code, lo_code + 1).astype(np.uint8)
    assert (codes == want).all()
    assert (codecs.e4m3_encode(-mid) == (want | 0x80)).all()
    # a hair either side of each midpoint goes to the nearer neighbour
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert (codecs.e4m3_encode(below) == lo_code).all()
    assert (codecs.e4m3_encode(above) == lo_code + 1).all()


def test_e4m3_encode_saturates_and_nan():
    x = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e6, np.inf, -449.0, -np.inf, np.nan, -np.nan])
    got = codecs.e4m3_encode(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x7F]


def test_e4m3_encode_subnormals_and_zero():
    tiny = 2.0 ** -9
    x = np.array([0.0, -0.0, tiny * 0.5, tiny * 0.5000001, tiny * 1.5, tiny * 2.5, tiny * 7.5, -tiny * 0.25, 1e-30])
    got = codecs.e4m3_encode(x)
    # 0.5 ulp ties to 0 (even); 1.5 -> 2; 2.5 -> 2; 7.5 -> 8 (= 2^-6, code 0x08); tiny negatives keep the sign
    assert list(got) == [0x00, 0x80, 0x00, 0x01, 0x02, 0x02, 0x08, 0x80, 0x00]


def test_e4m3_encode_vs_torch_after_clamp():
    rng = np.random.default_rng(7)
    mags = rng.standard_normal(200_000) * np.exp2(rng.uniform(-14, 10, 200_000))
    x32 = mags.astype(np.float32)
    ref = (torch.from_numpy(x32).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    ours = codecs.e4m3_encode(x32.astype(np.float64))
    assert (ours == ref).all()


# ---------------------------------------------------------------- f16 / bf16 / f32

def test_f16_decode_known_patterns():
    pats = {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14, 0x7BFF: 65504.0,
            0x3555: 0.333251953125, 0x8000: -0.0}
    for b, v in pats.items():
        assert codecs.f16_decode(np.array([b], np.uint16))[0] == v
    assert np.isnan(codecs.f16_decode(np.array([0x7E00], np.uint16))[0])
    assert codecs.f16_decode(np.array([0x7C00], np.uint16))[0] == np.inf


def test_f16_decode_all_vs_struct():
    b = np.arange(65536, dtype=np.uint16)
    ours = codecs.f16_decode(b)
    ref = np.array([struct.unpack("<e", struct.pack("<H", int(i)))[0] for i in range(65536)])
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and (ours[~nan] == ref[~nan]).all()


def test_bf16_decode_vs_struct_and_torch():
    b = np.arange(65536, dtype=np.uint16)
    ours = codecs.bf16_decode(b)
    ref = np.array([struct.unpack(">f", struct.pack(">HH", int(i), 0))[0] for i in range(65536)])
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and (ours[~nan] == ref[~nan]).all()
    tref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert (ours[~nan] == tref[~nan]).all()
    assert codecs.bf16_decode(np.array([0x3F80], np.uint16))[0] == 1.0


def test_f32_div_rn_is_correctly_rounded():
    # float64 quotient of binary32 operands, rounded once to binary32, is the
    # correctly rounded binary32 quotient (53 >= 2*24 + 2); struct does the rounding.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20_000) * 10).astype(np.float32)
    for s in (0.01, 0.0625, 0.0937, 0.1):
        s32 = float(np.float32(s))
        ours = codecs.f32_div_rn(x, s32)
        ref = np.array([struct.unpack("<f", struct.pack("<f", float(a) / s32))[0] for a in x], np.float32)
        assert (ours.view(np.uint32) == ref.view(np.uint32)).all()


def test_bits_dtype_and_decode_dispatch():
    assert codecs.bits_dtype("e4m3") == np.uint8
    with pytest.raises(ValueError):
        codecs.decode(np.zeros(1, np.uint8), "int4")


# ---------------------------------------------------------------- int8

def test_i8_decode_all_bytes_vs_struct():
    got = codecs.i8_decode(np.arange(256, dtype=np.uint8))
    want = [struct.unpack("<b", bytes([b]))[0] for b in range(256)]
    assert got.tolist() == [float(w) for w in want]


def test_i8_encode_ties_go_to_even_integers():
    for k in range(-127, 127):
        mid = k + 0.5
        even = k if k % 2 == 0 else k + 1
        got = codecs.i8_decode(codecs.i8_encode(np.array([mid])))[0]
        assert got == even, (mid, got)
        # just off the midpoint the nearer integer wins
        assert codecs.i8_decode(codecs.i8_encode(np.array([np.nextafter(mid, -np.inf)])))[0] == k
        assert codecs.i8_decode(codecs.i8_encode(np.array([np.nextafter(mid, np.inf)])))[0] == k + 1


def test_i8_encode_saturates_and_maps_nan_to_zero():
    x = np.array([127.49, 127.5, 128.0, 200.0, 1e30, np.inf, -127.49, -127.5, -128.0, -1e30, -np.inf, np.nan, -0.0,
                  -0.4, 0.5, -0.5])
    got = codecs.i8_decode(codecs.i8_encode(x)).tolist()
    assert got == [127, 127, 127, 127, 127, 127, -127, -127, -127, -127, -127, 0, 0, 0, 0, 0]
    # the byte -128 (0x80) is never produced
    assert 0x80 not in set(codecs.i8_encode(np.linspace(-300, 300, 100001)).tolist())


def test_i8_encode_matches_torch_round_and_clamp():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200000) * 60, np.arange(-130, 131) + 0.5])
    want = torch.clamp(torch.round(torch.from_numpy(x)), -127, 127).to(torch.int8).view(torch.uint8).numpy()
    assert np.array_equal(codecs.i8_encode(x), want)


def test_i8_cache_write_matches_torch_quantisation():
    """The oracle's cache write into INT8 equals torch's fp32 division, round
    half to even and clamp, for fp16 and bf16 sources."""
    import oracle
    rng = np.random.default_rng(12)
    for src, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        x = torch.from_numpy(rng.standard_normal((7, 3, 64)).astype(np.float32) * 3).to(tdt)
        x[0, 0, :4] = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0])
        bits = x.view(torch.int16).numpy().view(np.uint16)
        pool = np.zeros((2, 3, 8, 64), dtype=np.uint8)
        slots = np.arange(7)
        kc, vc = oracle.reshape_and_cache(bits, bits, pool, pool, slots, src, "i8", 0.037, 0.037)
        q = x.float() / torch.tensor(0.037, dtype=torch.float32)
        q = torch.where(torch.isnan(q), torch.zeros_like(q), q)
        want = torch.clamp(torch.round(q.clamp(-1e4, 1e4)), -127, 127).to(torch.int8).view(torch.uint8).numpy()
        got = kc.reshape(2, 3, 8, 64).transpose(0, 2, 1, 3).reshape(16, 3, 64)[:7]
        assert np.array_equal(got, want), src

"""Number formats of the KV cache, decoded and encoded from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Storage convention: a tensor of one of the five cache/query formats is handed
to the oracle as its raw bits, one unsigned integer per element:

======  ==================================  ============
name    format                              bits dtype
======  ==================================  ============
f32     IEEE 754 binary32                   uint32
f16     IEEE 754 binary16                   uint16
bf16    bfloat16 (upper half of binary32)   uint16
e4m3    OCP 8-bit float E4M3 ("E4M3FN")     uint8
i8      8-bit two's-complement integer      uint8
======  ==================================  ============

The pages name only "FP8" for the KV cache (page "vLLM-v0.17.1技术解析" §3.3
lists FP8 at 50% memory saving; the l189.com article §4 turns on an FP8 KV
cache).  The reading taken here is the OCP E4M3FN encoding with fp32 scales:
the stored byte encodes x / scale, and the cached value is decode(byte) *
scale, where the scale is the pool's one scale or, finer, the scale of the
row's head (one per head; the per-pool form is the case of equal scales).

The same pages list INT8 beside FP8 as an 8-bit format with the same 50%
memory saving ("vLLM-v0.17.1技术解析" §3.3), and the l189.com article §4
speaks of a quantised KV cache in "FP8 and similar formats".  The reading
taken for an INT8 KV cache mirrors the FP8 one: one fp32 scale per pool or
per head, stored byte = x / scale rounded to the nearest integer (ties to
even) and saturated to the symmetric range [-127, 127], cached value = byte *
scale.
INT8 has no NaN; a NaN input stores 0.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16", "e4m3", "i8")

# formats that hold x / scale with fp32 scales (per pool or per head)
SCALED = ("e4m3", "i8")

_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8, "i8": np.uint8}


def bits_dtype(name: str):
    """NumPy unsigned-integer dtype that carries the raw bits of format ``name``."""
    if name not in _BITS:
        raise ValueError(f"unknown format {name!r}")
    return _BITS[name]


# --------------------------------------------------------------------------
# decoders: raw bits -> exact float64 value
# --------------------------------------------------------------------------

def f32_decode(bits: np.ndarray) -> np.ndarray:
    """binary32 bits -> float64 (exact; NumPy reinterprets the bits)."""
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def f16_decode(bits: np.ndarray) -> np.ndarray:
    """binary16 bits -> float64 (exact; NumPy's float16 is IEEE binary16)."""
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float64.

    bfloat16 is the upper 16 bits of a binary32 word (sign, 8 exponent bits,
    7 fraction bits), so the value is that of the binary32 word whose lower
    16 bits are zero.
    """
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def _e4m3_value_of_code(code: int) -> float:
    """Value of one E4M3FN byte, from the format definition.

    Layout S.EEEE.MMM, exponent bias 7.  E = 0 encodes subnormals
    (-1)^S * M/8 * 2^-6; otherwise (-1)^S * (1 + M/8) * 2^(E-7).  The one
    pattern S.1111.111 is NaN; there is no infinity, so 1111 with M < 7 is
    an ordinary normal number (largest finite: 1.75 * 2^8 = 448).
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


# all 256 decodes, built once from the definition above
_E4M3_TABLE = np.array([_e4m3_value_of_code(c) for c in range(256)], dtype=np.float64)

# the 127 finite non-negative values, codes 0x00..0x7E, strictly increasing
_E4M3_POS = _E4M3_TABLE[:0x7F].copy()
E4M3_MAX = 448.0


def e4m3_decode(bits: np.ndarray) -> np.ndarray:
    """E4M3FN bytes -> float64 (exact; NaN for S.1111.111)."""
    return _E4M3_TABLE[np.asarray(bits, dtype=np.uint8)]


def i8_decode(bits: np.ndarray) -> np.ndarray:
    """INT8 bytes -> float64: the byte read as a two's-complement integer."""
    return np.asarray(bits, dtype=np.uint8).view(np.int8).astype(np.float64)


def decode(bits: np.ndarray, name: str) -> np.ndarray:
    """Raw bits of format ``name`` -> exact float64 values."""
    if name == "f32":
        return f32_decode(bits)
    if name == "f16":
        return f16_decode(bits)
    if name == "bf16":
        return bf16_decode(bits)
    if name == "e4m3":
        return e4m3_decode(bits)
    if name == "i8":
        return i8_decode(bits)
    raise ValueError(f"unknown format {name!r}")


# --------------------------------------------------------------------------
# encoders
# --------------------------------------------------------------------------

def f32_div_rn(x: np.ndarray, s) -> np.ndarray:
    """IEEE binary32 quotient x / s, rounded to nearest even, elementwise (s a
    number or an array that broadcasts against x).

    NumPy's float32 division is the IEEE operation on binary32 operands.
    """
    with np.errstate(all="ignore"):
        return np.asarray(x, dtype=np.float32) / np.asarray(s, dtype=np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Real values -> E4M3FN bytes: round to nearest, ties to even, saturating.

    * |x| above the largest finite value (448), infinities included, gives
      +-448 (sign kept); nothing finite becomes NaN.
    * NaN gives 0x7F.
    * Otherwise the nearest representable value is taken; at an exact
      midpoint the code with an even fraction field (an even byte, because
      codes 0x00..0x7E increase with the value) wins.  This covers the
      subnormal range (steps of 2^-9) and the rounding of tiny values to 0.
    * The sign bit of the input is kept, so -0.0 and negative values that
      round to zero give 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))

    # neighbours lo <= a <= hi in the table of finite non-negative values
    hi_idx = np.searchsorted(_E4M3_POS, a, side="left")  # first value >= a
    hi_idx = np.minimum(hi_idx, _E4M3_POS.size - 1)
    lo_idx = np.where(_E4M3_POS[hi_idx] == a, hi_idx, np.maximum(hi_idx - 1, 0))
    d_lo = a - _E4M3_POS[lo_idx]
    d_hi = _E4M3_POS[hi_idx] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_idx % 2 == 0))
    code = np.where(pick_hi, hi_idx, lo_idx).astype(np.uint8)

    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    return code


I8_MAX = 127


def i8_encode(x: np.ndarray) -> np.ndarray:
    """Real values -> INT8 bytes: nearest integer, ties to even, saturated to
    [-127, 127] (infinities included); NaN gives 0."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    r = np.rint(np.where(nan, 0.0, np.clip(x, -I8_MAX - 1.0, I8_MAX + 1.0)))   # NumPy rint: ties to even
    r = np.clip(r, -I8_MAX, I8_MAX)
    return r.astype(np.int8).view(np.uint8)

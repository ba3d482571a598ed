"""Storage codecs of the CPU oracle: OCP FP8 E4M3 ("e4m3fn"), bfloat16, and MXFP4.

TEST INFRASTRUCTURE ONLY. This module belongs to the oracle: it may be imported by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``,
and by nothing on the product path.

What the pages fix: a compressed KV entry keeps its RoPE dimensions in BF16 and the
rest in FP8 (researchpapers.dev explainer "DeepSeek V4 架构解读: CSA、HCA、mHC 与 Muon",
key-numbers table; PaperTrace analysis "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文", §2.5
and §3.3).  The pages do not name the FP8 variant; the reading taken here is OCP E4M3
(bias 7, no infinities, max 448, NaN = S.1111.111), unit scale, round to nearest with
ties to even, saturating to +-448.

The indexer's QK path may instead hold its keys and queries in MXFP4, the pages' later
revision of it (PaperTrace "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" §3.3: FP4 (MXFP4) on
the indexer's QK path, with 1x32 sub-blocks carrying their own scale factors).  The format is the OCP Microscaling (MX) v1.0
one: 32 elements share one E8M0 scale X = 2^(e - 127); each element is FP4 E2M1 (sign bit
3, exponent bits 2..1 with bias 1, mantissa bit 0; values 0, 0.5, 1, 1.5, 2, 3, 4, 6).
Encoding follows the MX conversion rule: X = 2^(floor(log2(max |v|)) - 2) (2 is E2M1's
largest exponent), then each v / X rounds to the nearest E2M1 value, ties to even,
saturating at +-6.  An all-zero block takes X = 1 (the rule leaves it open).  Two elements
share a byte: element 2i in the low nibble, 2i + 1 in the high one.

Rounding decisions are taken from the value first rounded to float32, because the kernels
produce their pre-storage values in float32: where floating point decides an integer code,
both sides decide from the same precision.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E4M3_MAX",
    "e4m3_values",
    "e4m3_decode",
    "e4m3_encode",
    "bf16_encode",
    "bf16_decode",
    "bf16_round_nearest",
    "to_f32",
    "E2M1_MAX",
    "e2m1_values",
    "e2m1_decode",
    "e2m1_encode_scaled",
    "e8m0_decode",
    "mxfp4_scale_exponent",
    "mxfp4_encode",
    "mxfp4_pack",
    "mxfp4_unpack",
    "mxfp4_decode",
]

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    """Value of every one of the 256 E4M3 codes, from the format's definition.

    sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent field 0 is
    subnormal: m/8 * 2^-6.  Codes 0x7f and 0xff are NaN; there is no infinity.
    """
    codes = np.arange(256)
    sign = codes >> 7
    expo = (codes >> 3) & 0xF
    mant = codes & 0x7
    mag = np.where(expo == 0, (mant / 8.0) * 2.0 ** -6, (1.0 + mant / 8.0) * 2.0 ** (expo - 7.0))
    val = np.where(sign == 1, -mag, mag).astype(np.float64)
    val[(expo == 0xF) & (mant == 0x7)] = np.nan
    return val


_E4M3 = _e4m3_table()
# Non-negative finite codes 0x00..0x7e in increasing order of value (0 .. 448).
_POS_CODES = np.arange(0x7F)
_POS_VALUES = _E4M3[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_values() -> np.ndarray:
    """A copy of the 256-entry decode table (float64, NaN for 0x7f/0xff)."""
    return _E4M3.copy()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8).astype(np.intp)]


def to_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def e4m3_encode(x) -> np.ndarray:
    """Values -> E4M3 codes (uint8): nearest code, ties to the even code, saturating at +-448.

    The input is first rounded to float32 (the precision the kernels decide in).  NaN maps
    to 0x7f.  The sign is kept, so a negative value that rounds to zero gives 0x80 (-0).
    """
    v = to_f32(x)
    nan = np.isnan(v)
    neg = np.signbit(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    exact = d_hi == 0
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


def bf16_encode(x) -> np.ndarray:
    """Values -> bfloat16 bit patterns (uint16), round to nearest even from float32.

    bfloat16 keeps the top 16 bits of a float32: the discarded low half is rounded with
    ties to even.  NaN maps to the quiet NaN 0x7fc0 with the input's sign.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    qnan = (((u >> 16) & 0x8000) | 0x7FC0).astype(np.uint16)
    return np.where(nan, qnan, r).astype(np.uint16)


def bf16_round_nearest(x) -> np.ndarray:
    """float64 values -> the nearest bfloat16 values (ties to even), rounded once from the
    float64 value itself (no float32 step, so no double rounding): with x = f 2^e, f in
    [0.5, 1), the 8 significant bits are rint(f 2^8) 2^(e - 8).  Used for the MXFP4
    indexer's BF16 scores, whose kernel rounds from an exact float64 sum."""
    x = np.asarray(x, np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- MXFP4

E2M1_MAX = 6.0
MX_BLOCK = 32


def _e2m1_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes: exponent field 0 is subnormal (m * 0.5), otherwise
    (1 + m / 2) * 2^(e - 1)."""
    codes = np.arange(16)
    sign = codes >> 3
    expo = (codes >> 1) & 0x3
    mant = codes & 0x1
    mag = np.where(expo == 0, mant * 0.5, (1.0 + mant / 2.0) * 2.0 ** (expo - 1.0))
    return np.where(sign == 1, -mag, mag).astype(np.float64)


_E2M1 = _e2m1_table()
_E2M1_POS = _E2M1[:8]
assert np.all(np.diff(_E2M1_POS) > 0)


def e2m1_values() -> np.ndarray:
    """A copy of the 16-entry E2M1 decode table (float64; code 8 is -0)."""
    return _E2M1.copy()


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64 values (exact)."""
    return _E2M1[np.asarray(codes, dtype=np.intp) & 0xF]


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale codes -> 2^(code - 127) (code 255 is NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, (c - 127).astype(np.int64)))


def e2m1_encode_scaled(x, e) -> np.ndarray:
    """Values x (rounded to float32 first) with the block exponent e (X = 2^e) -> E2M1 codes:
    x / X to the nearest E2M1 value, ties to the even code, saturating at +-6.  The sign is
    kept, so a negative value that rounds to zero gives code 8 (-0)."""
    v = to_f32(x)
    a = np.abs(v) / np.ldexp(1.0, np.asarray(e, dtype=np.int64))
    a = np.minimum(a, E2M1_MAX)
    hi = np.minimum(np.searchsorted(_E2M1_POS, a, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E2M1_POS[hi] - a
    d_lo = a - _E2M1_POS[lo]
    pick_hi = (d_hi == 0) | (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 8, code).astype(np.uint8)


def mxfp4_scale_exponent(x) -> np.ndarray:
    """Block exponents e (X = 2^e) of x [..., n], n a multiple of 32: floor(log2(max |v|)) - 2
    over each block of 32 float32-rounded values, 0 for an all-zero block, clamped to the
    E8M0 range [-127, 127]."""
    v = to_f32(x)
    blk = v.reshape(v.shape[:-1] + (v.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)           # amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1
    e = np.where(amax > 0, ex - 1 - 2, 0)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp4_encode(x):
    """Values x [..., n] -> (element codes uint8 [..., n], scale codes uint8 [..., n / 32])."""
    x = np.asarray(x, np.float64)
    e = mxfp4_scale_exponent(x)
    e_el = np.repeat(e, MX_BLOCK, axis=-1)
    return e2m1_encode_scaled(x, e_el), (e + 127).astype(np.uint8)


def mxfp4_pack(codes) -> np.ndarray:
    """Element codes [..., n] -> bytes [..., n / 2] (element 2i in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_unpack(packed) -> np.ndarray:
    """Bytes [..., n / 2] -> element codes [..., n]."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def mxfp4_decode(packed, scales) -> np.ndarray:
    """Packed element bytes [..., n / 2] and scale codes [..., n / 32] -> float64 [..., n]."""
    vals = e2m1_decode(mxfp4_unpack(packed))
    sc = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)
    return vals * sc

"""Storage codecs of the CPU oracle: OCP FP8 E4M3 ("e4m3fn") and bfloat16.

TEST INFRASTRUCTURE ONLY. This module belongs to the oracle: it may be imported by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``,
and by nothing on the product path.

What the pages fix: a compressed KV entry keeps its RoPE dimensions in BF16 and the
rest in FP8 (researchpapers.dev explainer "DeepSeek V4 架构解读: CSA、HCA、mHC 与 Muon",
key-numbers table; PaperTrace analysis "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文", §2.5
and §3.3).  The pages do not name the FP8 variant; the reading taken here is OCP E4M3
(bias 7, no infinities, max 448, NaN = S.1111.111), unit scale, round to nearest with
ties to even, saturating to +-448.

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
    "to_f32",
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


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)

"""Storage formats -> float64, the 8-bit float (e4m3) codec and the group-wise
8-bit integer codec.

The pages say an fp8 cache stores each number in one byte and fits about
twice the tokens (KV 缓存与分页注意力 §11; KV Cache内存优化技术原理与
PagedAttention分页注意力实现, "KV Cache量化压缩与多精度存储方案").  The
format used is OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, subnormals when the exponent field is 0, no infinities, and the single
NaN pattern S.1111.111; the largest finite magnitude is 448.  A per-tensor
fp32 scale maps stored codes back to values: value = e4m3(code) * scale, and
a value x is stored as e4m3(float32(x) * float32(1/scale)).

Encoding reading (where the pages are silent): clamp to [-448, 448] first
(saturating), then round to the nearest representable value with ties going
to the even mantissa; NaN stays NaN (0x7F with the sign); +-Inf saturate.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    """Value of one e4m3fn code, straight from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                                   # subnormal: m/8 * 2^(1-7)
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# magnitudes of the 127 non-negative finite codes 0x00..0x7E, strictly increasing
_MAGS = _TABLE[:0x7F].copy()


def e4m3_decode_table() -> np.ndarray:
    return _TABLE.copy()


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8): saturate, round half to even."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    nan = np.isnan(y)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")          # first magnitude >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _MAGS[hi], hi, code).astype(np.uint8)   # exact hits
    code = code | sign
    code = np.where(nan, np.uint8(0x7F) | sign, code)
    return code.astype(np.uint8)


INT8_MAX = 127


def int8_group_encode(x: np.ndarray):
    """float32 values [..., group] -> (int8 codes [..., group], float32 scales [...]).

    Group-wise symmetric 8-bit integers (KV Cache从原理到实战 §5.2: a scale per
    group of numbers, e.g. 128): here a group is one token's head vector.  In
    float32, as written: amax = max |x| over the group; scale = amax / 127;
    code = x / scale rounded to the nearest integer, ties to even, clamped to
    [-127, 127]; a group of zeros has scale 0 and codes 0.  Value = code * scale.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(INT8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (x / safe[..., None]).astype(np.float32)
    code = np.clip(np.rint(q), -INT8_MAX, INT8_MAX)
    code = np.where(scale[..., None] > 0, code, 0).astype(np.int8)
    return code, scale


def decode(a: np.ndarray, dtype: str, scale=1.0) -> np.ndarray:
    """Storage array -> float64 values (exact widening; fp8 times its scale; int8
    times its group's scale, ``scale`` then being an array of one scale per group,
    i.e. ``a.shape[:-1]``)."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float64)
    if dtype == "bf16":                       # bf16 = top half of an fp32
        bits = a.view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return _TABLE[a.view(np.uint8)] * float(scale)
    if dtype == "int8":
        return a.view(np.int8).astype(np.float64) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(dtype)

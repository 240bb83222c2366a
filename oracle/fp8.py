"""OCP 8-bit E4M3 codec for an fp8 KV cache (oracle).

The pages fix no fp8 format; this follows the OCP 8-bit floating point
specification's E4M3 encoding, the fp8 flavour native to CDNA4: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2**-9, no
infinities, the all-ones magnitude 0x7F is NaN, largest finite 448 (0x7E).

Encoding (a reading the pages leave open): y = fl32(x * inv_scale) with
inv_scale = fl32(1 / scale); NaN encodes as 0x7F with the sign of y; |y| >= 448
(infinities included) saturates to 448; otherwise y goes to the nearest code
value, ties to the code with an even mantissa. The sign bit of y is kept, also
when the magnitude rounds to zero. The encoder is brute force over all codes.

Per-head scales (an extension the pages do not cover: they fix no 8-bit format at all):
KV head h has its own scale, the per-tensor scale times a head factor (both float32
values, the product taken in float64); encode and decode then use that head's scale for
the head's elements. `scale` may be such an array, broadcast against the codes.

Pinned by: values fixed by the format definition, the round trip of every finite
code, and agreement with torch's independent float8_e4m3fn cast wherever that
cast does not overflow (tests/test_oracle_fp8.py).
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode_code(c: int) -> float:
    """Exact value of one E4M3 code."""
    c = int(c) & 0xFF
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# non-negative finite codes 0x00..0x7E and their values, ascending
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F]


def inv_scale_f32(scale):
    """fl32(1 / scale), elementwise for an array of scales."""
    if np.ndim(scale) == 0:
        return np.float32(1.0 / float(scale))
    return (1.0 / np.asarray(scale, dtype=np.float64)).astype(np.float32)


def head_scales(scale: float, head_factors) -> np.ndarray:
    """Per-head scales: the per-tensor scale times each head's factor, in float64."""
    return np.float64(np.float32(scale)) * np.asarray(head_factors, dtype=np.float32).astype(np.float64)


def encode_one(y: float) -> int:
    """Code for a float32 value y (already multiplied by inv_scale)."""
    y = float(np.float32(y))
    neg = math.copysign(1.0, y) < 0
    sign = 0x80 if neg else 0x00
    if math.isnan(y):
        return sign | NAN_CODE
    a = abs(y)
    if a >= MAX_FINITE:
        return sign | 0x7E
    d = np.abs(_POS_VALUES - a)
    best = d.min()
    cands = _POS_CODES[d == best]
    if len(cands) == 1:
        c = int(cands[0])
    else:
        even = [int(x) for x in cands if int(x) % 2 == 0]
        assert len(even) == 1, (y, cands)
        c = even[0]
    return sign | c


def encode(x, scale: float = 1.0) -> np.ndarray:
    """Encode an array of float32 (or exactly-float32) values with a per-tensor scale."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (x * inv_scale_f32(scale)).astype(np.float32)   # one float32 rounding
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    # brute force, memoised on the float32 bit pattern
    bits = flat.view(np.uint32)
    uniq, inv = np.unique(bits, return_inverse=True)
    codes = np.array([encode_one(float(b)) for b in uniq.view(np.float32)], dtype=np.uint8)
    out[:] = codes[inv]
    return out.reshape(y.shape)


def decode(codes, scale=1.0) -> np.ndarray:
    """Exact float64 values of codes, times the scale (per tensor, or an array broadcast
    against the codes)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)

"""FP8 E4M3 (OCP "fn" variant) encoding of KV values, from its definition.

TEST INFRASTRUCTURE ONLY (see the package header): the GPU path never
imports this module.

[DISAGG] "布局转换" lists a dtype change among the conversions done around
a KV transfer (one side BF16 KV, the other FP8 KV).  The pages fix neither
the FP8 format nor the scaling; the reading taken here is the OCP E4M3 "fn"
format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; no
infinities; exponent 15 with mantissa 7 is NaN, so the largest finite value
is 1.75 * 2^8 = 448; subnormals m * 2^-9) with one scale per tensor: the
stored value encodes ``fp32(x) * inv`` with ``inv = fp32(1 / scale)`` (both
IEEE fp32 operations), clamped to [-448, 448] and rounded to the nearest
representable value, ties to an even mantissa.  Decoding multiplies back by
the scale.

Everything is written with exact float64 arithmetic on the fp32 quotient:
every fp32 value and every E4M3 value is exact in float64.
"""

from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0
NAN_BITS = 0x7F


def _round_half_even(x: float) -> int:
    f = math.floor(x)
    d = x - f
    if d > 0.5 or (d == 0.5 and f % 2 == 1):
        return f + 1
    return f


def encode_value(x: float) -> int:
    """E4M3 bits of one finite value (already divided by the scale), clamped to +-448."""
    if math.isnan(x):
        return NAN_BITS
    sign = 0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0
    a = min(abs(x), MAX_FINITE)
    if a < 2.0 ** -6:                                      # subnormal (or zero): multiples of 2^-9
        q = _round_half_even(a / 2.0 ** -9)                # 8 here is the smallest normal, bits 0x08
        return sign | q
    e = math.floor(math.log2(a))
    # guard against log2 rounding at exact powers of two
    if 2.0 ** e > a:
        e -= 1
    elif 2.0 ** (e + 1) <= a:
        e += 1
    q = _round_half_even((a / 2.0 ** e - 1.0) * 8.0)
    if q == 8:
        e, q = e + 1, 0
    if e > 8 or (e == 8 and q == 7):                       # above 448 (cannot happen after the clamp)
        e, q = 8, 6
    return sign | ((e + 7) << 3) | q


def decode_value(bits: int) -> float:
    """The value an E4M3 byte holds (NaN for the two NaN patterns)."""
    bits &= 0xFF
    sign = -1.0 if bits & 0x80 else 1.0
    e, m = (bits >> 3) & 0xF, bits & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def inverse_scale(scale: float) -> np.float32:
    """fp32(1 / scale), one IEEE fp32 division."""
    return np.float32(np.float32(1.0) / np.float32(scale))


def quantize(values_f32: np.ndarray, scale: float) -> np.ndarray:
    """uint8 E4M3 bits of fp32(values) * fp32(1 / scale) (IEEE fp32 product), element by element."""
    v = np.asarray(values_f32, dtype=np.float32)
    with np.errstate(all="ignore"):
        q = (v * inverse_scale(scale)).astype(np.float32)  # one IEEE fp32 product per element
    flat = q.ravel()
    out = np.empty(flat.size, dtype=np.uint8)
    for i in range(flat.size):
        out[i] = encode_value(float(flat[i]))
    return out.reshape(v.shape)


def dequantize(bits: np.ndarray, scale: float) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint8)
    return np.array([decode_value(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape) * scale


_TABLES: dict = {}


def quantize_bf16(bits_u16: np.ndarray, scale: float) -> np.ndarray:
    """quantize() for bfloat16 inputs given as raw uint16 bits: the 65536 possible inputs are encoded once per
    scale with encode_value and looked up (same results as quantize, fast enough for whole pools)."""
    key = float(np.float32(scale))
    tab = _TABLES.get(key)
    if tab is None:
        allv = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
        tab = quantize(allv, scale)
        _TABLES[key] = tab
    return tab[np.asarray(bits_u16, dtype=np.uint16)]

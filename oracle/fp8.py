"""OCP FP8 E4M3 (the "fn" variant) code table and conversions.  TEST INFRASTRUCTURE ONLY.

Format (OCP 8-bit Floating Point Specification, OFP8, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
S.1111.111 is NaN; there are no infinities; the largest finite magnitude is
S.1111.110 = 448.  The long-context workload stores its KV pool in this format with
one float32 scale per (kv-head, K or V) (deployment-tuning page, KV cache dtype
option fp8_e4m3).

Quantisation reading: code = round-to-nearest-even(fp32(x * inv_scale)) on the
E4M3 grid, saturating to +-448; dequantised value = decode(code) * scale.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_code(code: int) -> float:
    """Value of one E4M3 code (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# the 127 non-negative finite values, ascending with their codes (codes 0x00..0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = np.array([decode_code(c) for c in range(0x7F)], dtype=np.float64)
assert np.all(np.diff(_POS_VALUES) > 0)

DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def encode(x) -> np.ndarray:
    """Round finite values to the nearest E4M3 code, ties to the even code, saturating at 448.

    ``x`` is taken as float64 exactly (callers pass float32 products)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8 oracle encoder takes finite values only")
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the first grid value >= a
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo = _POS_VALUES[lo]
    vhi = _POS_VALUES[hi]
    dlo = a - vlo
    dhi = vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0))
    idx = np.where(a >= vhi, hi, np.where(pick_hi, hi, lo))
    code = _POS_CODES[idx]
    # the sign bit is kept, so negative values that round to zero give -0 (0x80)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantise(x_f32: np.ndarray, inv_scale: np.ndarray) -> np.ndarray:
    """E4M3 codes of fp32(x * inv_scale); ``inv_scale`` broadcasts over x (float32)."""
    prod = (np.asarray(x_f32, dtype=np.float32) * np.asarray(inv_scale, dtype=np.float32)).astype(np.float32)
    return encode(prod)


def dequantise(codes: np.ndarray, scale) -> np.ndarray:
    """float64 code value times scale (exact in float64)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.int64)] * np.asarray(scale, dtype=np.float64)

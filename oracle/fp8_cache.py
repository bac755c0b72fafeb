"""fp8 (e4m3) retrieval KV cache and the values attention sees (test oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

The pages tie DuoAttention's 3.3-million-token context to combining it with
quantization (abstract on the pith.science review page) and name no scheme.
This module is the second scheme the library offers (the first is int8,
``quantized_cache``).  Readings:

E1. Only retrieval heads' K and V rows are stored as fp8; streaming caches
    stay bf16.
E2. The format is the OCP 8-bit float E4M3 ("e4m3fn"): 1 sign bit, 4
    exponent bits (bias 7), 3 mantissa bits, subnormals, no infinities; the
    largest finite magnitude is 448 and codes 0x7F / 0xFF are NaN.
E3. One scale per tensor (K, and V) for the whole cache, a power of two set
    in the configuration, so that dividing by it is exact: code =
    e4m3(x / scale) where e4m3() clamps to [-448, 448] and rounds to the
    nearest representable value, ties to an even mantissa; a zero keeps its
    sign.  The stored value is code * scale.
E4. Every K and V row a call attends to -- rows of earlier calls and the
    call's own new rows alike -- is seen through its stored value: the
    library stores a call's rows before it attends.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    """Value of every code 0..255 (NaN for 0x7F and 0xFF), from the format's
    definition."""
    out = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * m * 2.0 ** -9  # subnormal: m/8 * 2^(1-7)
        else:
            out[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Clamp to [-448, 448] and round to nearest, ties to an even mantissa
    (reading E3).  x: any real array (no NaN).  Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no e4m3 encoding here")
    a = np.minimum(np.abs(x), E4M3_MAX)
    pos_codes = np.arange(0x7F)  # 0x00 .. 0x7E: the non-negative finite values, increasing
    pos_vals = E4M3_VALUES[pos_codes]
    hi = np.searchsorted(pos_vals, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(pos_vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - pos_vals[lo], pos_vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo]).astype(np.uint8)
    code = np.where(a == pos_vals[hi], pos_codes[hi], code).astype(np.uint8)  # exact values
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_rows_fp8(x, scale: float) -> np.ndarray:
    """Codes of the rows of x (reading E3); scale a power of two."""
    m, e = np.frexp(scale)
    if m != 0.5:
        raise ValueError("the scale must be a power of two")
    return e4m3_encode(np.asarray(x, dtype=np.float64) / scale)


def dequantize_rows_fp8(codes, scale: float) -> np.ndarray:
    return e4m3_decode(codes) * scale


def seen_rows_fp8(x_seq, retrieval: bool, scale: float) -> np.ndarray:
    """The K (or V) values one (sequence, KV head) is attended through
    (readings E1, E4): every row of a retrieval head through its fp8 code,
    streaming heads as given.  float64 [T, D]."""
    x = np.asarray(x_seq, dtype=np.float64)
    if not retrieval:
        return x.copy()
    return dequantize_rows_fp8(quantize_rows_fp8(x, scale), scale)

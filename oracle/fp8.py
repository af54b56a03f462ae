"""Per-row e4m3 quantization of the query, for the fp8-arithmetic attention.

Test infrastructure only (see the package docstring).

The pages count numeric precision (FP8 / FP4) among what decides real
serving speed (Aurora, everytik.com and chernovdev.ru mirrors, section 1, on
acceptance rate versus speed-up).  The fp8-arithmetic attention feeds the
query to the fp8 matrix cores, so each (node, head) row of q is first
rounded to OCP e4m3.  Reading (the pages give no recipe), in float32 steps:

    amax  = max |q[row]|                         (rows of zeros: scale 1)
    codes = round_to_nearest_even_e4m3(q[row] * (448 / amax))
    scale = amax * (1 / 448)
    q_hat = codes * scale                         (what the products see)

Encoding is written from the format's definition: the value is rounded to
the nearest of the 253 finite e4m3 values, a tie going to the code with an
even mantissa (the even code).  In float32, q * (448 / amax) can exceed 448
by an ulp; it rounds to 448 (the kernel clamps to +-448, the same value).
"""
from __future__ import annotations

import numpy as np

from .attention import e4m3_decode_table

_TAB = e4m3_decode_table()
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)       # 0x00 .. 0x7E: +0 .. +448
_POS_VALS = _TAB[_POS_CODES]


def encode_e4m3(x) -> np.ndarray:
    """float values (|x| < 464) -> uint8 e4m3 codes, round to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) >= 464.0) or not np.all(np.isfinite(x)):
        # below 464 (half-way to the next binade step above 448) the nearest
        # value is at most 448; nothing here produces larger magnitudes
        raise ValueError("e4m3 encoding here takes finite values with |x| < 464")
    a = np.abs(x).ravel()
    hi = np.searchsorted(_POS_VALS, a, side="left")                     # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(_POS_CODES[lo] % 2 == 0, lo, hi), pick)
    code = _POS_CODES[pick]
    neg = (x.ravel() < 0) & (code != 0)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8).reshape(x.shape)


def quantize_rows_e4m3(q) -> tuple[np.ndarray, np.ndarray]:
    """q [..., D] (values exact in float32) -> (codes uint8 [..., D], scale
    float32 [...]) by the recipe above, every step in float32."""
    q32 = np.asarray(q, dtype=np.float32)
    amax = np.max(np.abs(q32), axis=-1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(448.0) / safe).astype(np.float32)
    scaled = (q32 * inv[..., None]).astype(np.float32)
    codes = encode_e4m3(scaled.astype(np.float64))
    scale = np.where(zero, np.float32(1.0), (safe * np.float32(1.0 / 448.0)).astype(np.float32)).astype(np.float32)
    return codes, scale


def dequantize_rows_e4m3(codes, scale) -> np.ndarray:
    """codes * scale in float64 (exact: 4 significant bits times a float32)."""
    return _TAB[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)[..., None]

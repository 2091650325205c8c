"""Per-token fp8 (OCP e4m3fn) quantisation of indexer inputs.

The pages give the long-context configuration's indexer inputs as fp8 e4m3
values with per-token fp32 scales, but not the quantiser that makes them. This
library's reading, computed here with binary32 (NumPy float32) decisions:

    amax_r  = max_c |x[r, c]|                         (exact)
    scale_r = fl32(amax_r / 448)      (1 when amax_r == 0)
    y       = fl32(x[r, c] / scale_r)
    code    = the e4m3fn value nearest to y, ties to the even mantissa, with
              magnitudes above 448 clamped to 448; the sign bit is y's

fl32 is IEEE-754 binary32 round-to-nearest-even. 448 is the largest finite
e4m3fn magnitude (OCP 8-bit Floating Point Specification), so each row's
largest element maps to +-448 and dequantisation is code * scale_r.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3fn_table

_MAG = e4m3fn_table()[:0x7F]  # magnitudes of codes 0x00 .. 0x7E, increasing


def e4m3fn_encode(y) -> np.ndarray:
    """Codes (uint8) of the e4m3fn values nearest to the float32 values y
    (ties to the even mantissa; |y| > 448 clamps to 448; sign from y)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    hi = np.searchsorted(_MAG, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, len(_MAG) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAG[lo]
    d_hi = _MAG[hi] - a
    # nearer neighbour; on a tie the even code (its lowest bit is the mantissa's)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return (code | np.where(np.signbit(y), 0x80, 0x00).astype(np.uint8)).astype(np.uint8)


def quantize_rows_fp8(x_bits):
    """x_bits: uint16 bf16 bit patterns [rows, cols]. Returns (codes uint8
    [rows, cols], scales float32 [rows])."""
    x = bf16_to_f64(np.asarray(x_bits)).astype(np.float32)   # bf16 -> f32 is exact
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    amax = np.max(np.abs(x), axis=1)
    scale = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    scale = scale.astype(np.float32)
    y = (x / scale[:, None]).astype(np.float32)
    return e4m3fn_encode(y), scale

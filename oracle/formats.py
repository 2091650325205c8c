"""Decoding of the device input formats, written from the format definitions.

bfloat16: the upper 16 bits of an IEEE-754 binary32, so a bf16 value is exactly
the binary32 whose high half is the stored bits and whose low half is zero.

OCP fp8 E4M3 ("e4m3fn", OCP 8-bit Floating Point Specification v1.0): 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2**-6; there are no infinities; the codes with exponent 15 and
mantissa 7 (0x7F, 0xFF) are NaN; the largest finite magnitude is 448.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 values of an array of raw bfloat16 bit patterns (uint16)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 input must be given as uint16 bit patterns")
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3fn codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (-6)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3 = e4m3fn_table()


def e4m3fn_to_f64(codes) -> np.ndarray:
    """Exact float64 values of an array of raw e4m3fn codes (uint8)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("fp8 input must be given as uint8 codes")
    return _E4M3[c]

"""Exact decoding of stored number formats to float64 (oracle side).

bfloat16: the upper 16 bits of an IEEE binary32; decoding shifts the bits back.
fp8 E4M3 "fn" (OCP 8-bit floating point, the format the FlashRec deployment guide names as
its fp8_e4m3 KV cache, "precision and memory" section): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; there
is no infinity; the largest finite value is 448.
"""
from __future__ import annotations

import numpy as np


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3fn_table() -> np.ndarray:
    t = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * 2.0 ** -6 * (m / 8.0)
        else:
            t[code] = sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return t


_E4M3FN = _e4m3fn_table()


def decode_e4m3fn_bits(bits: np.ndarray) -> np.ndarray:
    return _E4M3FN[np.asarray(bits, dtype=np.uint8)]


def decode_stored(x: np.ndarray, dtype: str, scale=None) -> np.ndarray:
    """Stored tensor -> float64 values.  ``scale`` multiplies fp8 codes (broadcast)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16_bits(x)
    if dtype == "fp8":
        v = decode_e4m3fn_bits(x)
        return v if scale is None else v * np.asarray(scale, dtype=np.float64)
    raise ValueError(dtype)

"""Decode stored KV / query bytes to float64 (oracle; test infrastructure only).

bf16: the upper 16 bits of an IEEE-754 binary32; decoding shifts the payload
left by 16 and reads the word as binary32, then widens to float64.

e4m3fn (OCP 8-bit float, "FN" = finite-only): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits.  Exponent field 0 encodes subnormals m/8 * 2^-6;
exponent fields 1..15 encode (1 + m/8) * 2^(e-7), except S.1111.111 which is
NaN.  There is no infinity; the largest finite magnitude is 448.

The per-token scale of the e4m3 KV format is one float32 per latent row; the
decoded value is code_value * scale, formed here in float64.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray, scale=None) -> np.ndarray:
    """Decode e4m3fn codes; multiply each row by its float32 scale if given."""
    v = E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]
    if scale is not None:
        v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    return v


def decode_rows(data: np.ndarray, scale=None) -> np.ndarray:
    """Latent rows in either stored format -> float64 [n][576]."""
    data = np.asarray(data)
    if data.dtype == np.uint16:
        return bf16_to_f64(data)
    if data.dtype == np.uint8:
        return e4m3_to_f64(data, scale)
    raise TypeError(f"unsupported stored dtype {data.dtype}")

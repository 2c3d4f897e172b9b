"""Decoding of stored element types, written from the formats' definitions.

bf16: the upper 16 bits of an IEEE binary32; value = float32 with those bits and a
zero lower half.

fp8 E4M3FN (OCP 8-bit floating point, E4M3 variant without infinities): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 is subnormal,
value = (-1)^s * (m / 8) * 2^-6; otherwise value = (-1)^s * (1 + m / 8) * 2^(e - 7).
Exponent 15 with mantissa 7 is NaN; there is no infinity; the largest finite value
is 448.  The pages name FP8 storage for the dense draft layer ([PR18066] view-scale
commit); one float32 scale per tensor multiplies the decoded value.
"""
import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """float64 values of E4M3FN bytes (NaN for the two NaN codes)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def decode_store(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Unscaled float32 values of a stored array ('f32', 'bf16' bits, 'fp8' bits).
    Every bf16 and E4M3FN value is exactly representable in float32."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "fp8":
        return decode_e4m3fn(raw).astype(np.float32)
    raise ValueError(dtype)

"""Widen stored K/V/Q values to float64 exactly (test oracle).

bf16 is the top half of an IEEE binary32; widening appends sixteen zero bits.

fp8 e4m3 (OCP "e4m3fn" form, the fp8 KV-cache format named in "Track C ·
Document 10 · Shrinking the footprint", fp8 section) packs sign | 4 exponent
bits | 3 mantissa bits with exponent bias 7:

* exponent field 0: subnormal, value (-1)^s * (m / 8) * 2^-6;
* otherwise        : (-1)^s * (1 + m / 8) * 2^(e - 7);
* the all-ones pattern s.1111.111 is NaN; there is no infinity, so the
  largest finite magnitude is (1 + 6/8) * 2^8 = 448.

A stored fp8 code decodes to ``code_value * scale`` with one float32 scale per
KV head (separate for K and V).
"""
import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return np.asarray(bits).astype(np.int32).view(np.float32).astype(np.float64)


def fp8_e4m3_value(code: int) -> float:
    """Decode one fp8 e4m3fn code (0..255) from its bit fields."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


FP8_E4M3_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp8_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return FP8_E4M3_TABLE[np.asarray(bits).astype(np.uint8)]


def stored_to_f64(bits: np.ndarray, dtype: str, scale=None) -> np.ndarray:
    """Stored bits of a ``[..., H_kv, d]`` (or ``[..., d]``) array to float64.

    ``scale`` (fp8 only) is indexed by the second-to-last axis: one factor per
    KV head.
    """
    if dtype == "f32":
        return f32_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "fp8":
        x = fp8_bits_to_f64(bits)
        if scale is not None:
            x = x * np.asarray(scale, np.float64)[:, None]
        return x
    raise ValueError(dtype)

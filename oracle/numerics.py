"""Number formats used by the oracle -- test infrastructure only.

BF16 is 1 sign bit, 8 exponent bits and 7 fraction bits; FP32 has 23 fraction
bits.  Conversion to BF16 keeps the top 16 bits of the FP32 pattern and rounds
to nearest, ties to even, with everything below the rounding bit acting as the
sticky bit (paper-graph-ui summary of arXiv 2510.04212, section 3.4.4, "The BF16
addition mechanism" and the concrete bit-level example).

All functions work on numpy arrays and return new arrays.  Pinned by
tests/test_oracle_numerics.py against the printed worked example and against a
brute-force nearest-value search.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


def f32(x) -> np.ndarray:
    """Round (float64) values to the nearest FP32 value (ties to even)."""
    return np.asarray(x, dtype=F64).astype(F32)


def f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=F32)).view(np.uint32)


def f32_from_bits(bits) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(bits, dtype=np.uint32)).view(F32)


def bf16_rne(x) -> np.ndarray:
    """FP32 -> BF16 with round to nearest, ties to even; result stored as FP32.

    The kept part is the top 16 bits.  Adding 0x7FFF plus the lowest kept bit
    to the pattern carries into the kept part exactly when the dropped part is
    above the halfway point, or at it with an odd kept part.  NaN stays NaN;
    values that round past the largest finite BF16 become infinity.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    u = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(F32).copy()
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out.reshape(a.shape)


def bf16_bits(x) -> np.ndarray:
    """The 16-bit BF16 pattern of values that are already BF16-representable."""
    return (f32_bits(x) >> np.uint32(16)).astype(np.uint16)


def is_bf16(x) -> np.ndarray:
    """True where the FP32 value is exactly representable in BF16."""
    return (f32_bits(x) & np.uint32(0xFFFF)) == 0


def split_hi_lo(p) -> tuple[np.ndarray, np.ndarray]:
    """Two-term BF16 expansion of an FP32 value: hi = bf16(p), lo = bf16(p - hi).

    p - hi is exact in FP32 (hi is p with its low 16 bits changed by at most one
    BF16 ulp), so hi + lo carries 16 significant bits of p.  This is the
    high-precision P-bar the FP32-output remedy multiplies V with.
    """
    p = np.asarray(p, dtype=F32)
    hi = bf16_rne(p)
    lo = bf16_rne((p - hi).astype(F32))
    return hi, lo


def bf16_ulp(x) -> np.ndarray:
    """Spacing of BF16 values at |x| (normal range): 2**(exponent(x) - 7)."""
    x = np.abs(np.asarray(x, dtype=F64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, np.exp2(e - 7), 0.0)


def f32_ulp(x) -> np.ndarray:
    """Spacing of FP32 values at |x| (normal range): 2**(exponent(x) - 23)."""
    x = np.abs(np.asarray(x, dtype=F64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, np.exp2(e - 23), 0.0)

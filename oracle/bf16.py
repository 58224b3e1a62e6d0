"""bfloat16 encode/decode for the oracle, written from the IEEE-754 definition.

bfloat16 = the top 16 bits of an IEEE binary32: 1 sign bit, 8 exponent bits (bias
127), 7 stored fraction bits (8 significant bits with the hidden bit).  Subnormals
have a quantum of 2^-133.  Rounding is to nearest, ties to even.

These routines do NOT go through float32: rounding is done once, directly from the
float64 value, so the oracle never double-rounds.  They are pinned (tests) against
torch's CPU float32 -> bfloat16 conversion on fp32-representable values and on
hand-built ties, subnormals, overflow and NaN.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX_EXP = 128          # values >= 2^128 after rounding overflow to inf
_BF16_MIN_QUANTUM = 2.0 ** -133


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); return uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    fin = np.isfinite(x)
    # exponent of each value: |x| = mant * 2^e with mant in [0.5, 1)
    _, e = np.frexp(np.where(fin, x, 0.0))
    # quantum (spacing of bf16 numbers around x): 8 significant bits, floored at the
    # subnormal quantum 2^-133
    q = np.maximum(np.ldexp(1.0, e - 8), _BF16_MIN_QUANTUM)
    r = np.where(fin, np.round(np.where(fin, x, 0.0) / q) * q, x)   # np.round: half to even
    over = fin & (np.abs(r) >= 2.0 ** _BF16_MAX_EXP)
    r = np.where(over, np.copysign(np.inf, x), r)
    # r is now exactly representable in bf16 (or +-inf), hence in float32
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[...] = bits
    out[nan] = 0x7FC0
    return out


def f32_round(x) -> np.ndarray:
    """Round float64 values to float32 (numpy's conversion: nearest, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)

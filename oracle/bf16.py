"""bf16 codec of the oracle (test infrastructure only).

bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits,
7 stored significand bits (8 significant bits for normal numbers), smallest
normal 2^-126, subnormal spacing 2^-133.  Every bf16 value is exactly a
float64, so decoding is exact; encoding rounds a float64 *directly* to bf16
(round to nearest, ties to even) -- never through float32, which would round
twice.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = float(np.ldexp(255.0, 120))   # 0x7F7F = (2 - 2^-7) * 2^127
_EMIN_Q = -125                            # frexp exponent where the spacing stops shrinking


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):       # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def _quantum(v: np.ndarray) -> np.ndarray:
    """Exponent of the bf16 spacing at |v|: v = m * 2^e with 0.5 <= |m| < 1 has
    spacing 2^(e - 8) for normal bf16, and 2^-133 below 2^-126."""
    _, e = np.frexp(v)
    return np.maximum(e, _EMIN_Q) - 8


def f64_round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    Overflow past the rounding threshold of the largest finite bf16 gives inf;
    NaN stays NaN."""
    v = np.asarray(v, dtype=np.float64)
    q = _quantum(v)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)   # np.rint rounds half to even
    big = np.abs(r) > _BF16_MAX
    r = np.where(big, np.copysign(np.inf, v), r)
    r = np.where(np.isinf(v), v, r)
    return np.where(np.isnan(v), np.nan, r)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one RNE rounding; NaN -> 0x7FC0."""
    r = f64_round_bf16(v)
    nan = np.isnan(r)
    r32 = np.where(nan, 0.0, r).astype(np.float32)   # exact: r is a bf16 value
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), bits)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v|: 2^(floor(log2|v|) - 7) for normal
    magnitudes, 2^-133 at and below the subnormal range (and for v = 0)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.where(v == 0, _EMIN_Q, e)            # frexp(0) reports exponent 0
    return np.ldexp(1.0, np.maximum(e, _EMIN_Q) - 8)

"""bf16 round-to-nearest-even from fp64, and bf16 bit patterns to fp64.

bf16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits, 7
stored mantissa bits.  Rounding is done directly from fp64 (one rounding, no
detour through fp32), ties to even, with gradual underflow (no flush to
zero) and overflow to infinity.
"""

from __future__ import annotations

import numpy as np

_MIN_NORMAL = 2.0 ** -126
_SUB_QUANTUM_EXP = -133  # bf16 subnormal spacing is 2**-133
_OVERFLOW = 2.0 ** 128


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each element, returned as fp64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(x)  # x = m * 2**e with 0.5 <= |m| < 1
        normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        sub = np.ldexp(np.rint(np.ldexp(x, -_SUB_QUANTUM_EXP)), _SUB_QUANTUM_EXP)
        r = np.where(np.abs(x) < _MIN_NORMAL, sub, normal)
        r = np.where(np.abs(r) >= _OVERFLOW, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
    return r


def to_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of the RNE rounding of ``x``; NaN -> 0x7FC0."""
    r = round_bf16(x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(r), np.uint16(0x7FC0), bits).astype(np.uint16)


def from_bits(bits) -> np.ndarray:
    """fp64 values of bf16 bit patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)

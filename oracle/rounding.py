"""Rounding of float64 results to the output dtypes (oracle; test infrastructure only).

The pages fix no rounding mode; the reading taken is IEEE round-to-nearest-even, applied
once, from the float64 result straight to the output dtype.
"""

import numpy as np

# bfloat16: 8 significant bits (7 stored), exponent range of float32.
_BF16_SIG_BITS = 8
_BF16_MIN_QUANTUM_EXP = -133  # subnormal spacing 2**-126 * 2**-7
_BF16_OVERFLOW = 2.0 ** 128


def round_bf16(y):
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    ``frexp`` gives y = m * 2**e with 0.5 <= |m| < 1, so the bf16 quantum at y is
    2**(e - 8), floored at the subnormal quantum. Scaling by a power of two and ``rint``
    (ties to even) are exact in float64, so there is a single rounding. Magnitudes that
    round to 2**128 or beyond become infinities; NaN and infinities pass through; the sign
    of zero is kept.
    """
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)
    q = np.maximum(e.astype(np.int64) - _BF16_SIG_BITS, _BF16_MIN_QUANTUM_EXP)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.ldexp(np.rint(np.ldexp(y, -q)), q)
        r = np.where(np.abs(r) >= _BF16_OVERFLOW, np.copysign(np.inf, y), r)
    return np.where(np.isfinite(y), r, y)


def round_f32(y):
    """float64 -> nearest float32 (IEEE cast, ties to even), returned as float64."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(y, dtype):
    """Round a float64 result to ``dtype`` in {"bf16", "f32"}; "f64" leaves it unrounded."""
    if dtype == "bf16":
        return round_bf16(y)
    if dtype == "f32":
        return round_f32(y)
    if dtype == "f64":
        return np.asarray(y, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits(v):
    """Bit patterns (uint16) of float64 values that are already bf16 values."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (v32.view(np.uint32) >> 16).astype(np.uint16)


def f32_param(v):
    """The exact float32 value of a parameter the pages store as ``f32::to_bits``."""
    return float(np.float32(v))

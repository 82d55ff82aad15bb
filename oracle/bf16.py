"""bf16 <-> float64 at the bit level (test infrastructure only).

bf16 is the top half of an IEEE float32: 1 sign, 8 exponent, 7 mantissa bits.
Widening is exact; narrowing rounds to nearest with ties to even.  NumPy has
no bf16 type, so values travel as uint16 bit patterns.
"""

import numpy as np


def to_f64(bits) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def from_f64(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); return bits.

    Rounds directly from float64 (no intermediate float32, so no double
    rounding).  Values must be finite and inside the bf16 normal range or
    zero/subnormal.  ``np.rint`` rounds exact halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x8000, 0).astype(np.int64)
    a = np.abs(x)
    m, e = np.frexp(a)                      # a = m * 2**e with 0.5 <= m < 1
    e = e.astype(np.int64)
    normal = (e - 1) >= -126
    n = np.rint(m * 256.0).astype(np.int64)  # 8 significant bits, in [128, 256]
    carry = n == 256
    n = np.where(carry, 128, n)
    e = np.where(carry, e + 1, e)
    bits_normal = ((e - 1 + 127) << 7) | (n - 128)
    sub = np.rint(np.where(normal, 0.0, a) * 2.0 ** 133).astype(np.int64)  # subnormal spacing 2**-133
    bits = np.where(a == 0, 0, np.where(normal, bits_normal, sub))
    return (sign | bits).astype(np.uint16)


def ulp(bits) -> np.ndarray:
    """Spacing of bf16 values at each given bf16 value (float64)."""
    b = np.asarray(bits, dtype=np.uint16)
    e = ((b >> 7) & 0xFF).astype(np.int64)
    e = np.maximum(e, 1)
    return np.ldexp(1.0, e - 127 - 7)

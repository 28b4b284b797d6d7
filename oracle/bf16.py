"""bfloat16 bit-pattern conversions for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32: widening is a 16-bit
shift and is exact; narrowing rounds to nearest, ties to even (RNE), with NaN
kept NaN (quieted).  Both pages that fix output precision round once, at the
end, to bf16 (MaxText PR #5760, commit on valid rows: the GLU keeps float32
throughout and narrows its result a single time).
"""

import numpy as np


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32, exactly (shift into the high half)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64, exactly (every bf16 is a float64)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def f32_to_bf16_bits(x):
    """float32 -> uint16 bf16 bits, round to nearest even; NaN stays NaN.

    Finite values: add 0x7FFF plus the lowest kept bit, then drop the low 16
    bits (the classic integer form of RNE).  Overflow past the largest bf16
    lands on the infinity pattern, as IEEE rounding requires.  NaNs keep their
    sign and top payload bits and get the quiet bit set.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    is_nan = (b & 0x7FFFFFFF) > 0x7F800000
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    quiet = (b >> 16) | 0x0040
    out = np.where(is_nan, quiet, rounded) & 0xFFFF
    return out.astype(np.uint16)

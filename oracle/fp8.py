"""fp8 (OCP E4M3) decoding and the fp8 ragged_dot (test infrastructure only).

SkyRL-tx PR #867 ("Integrate ragged_dot pallas kernel with group_offset
support") parametrises the kernels by a compute dtype and reports results
only for bf16; the fp8 form here is the plainest reading: OCP FP8 E4M3
inputs, the exact products accumulated (here in float64), no scaling.

E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
field 0 holds the subnormals m/8 * 2^-6; otherwise the value is
(1 + m/8) * 2^(e-7); the pattern S.1111.111 is NaN and there is no
infinity, so the largest magnitude is 448.  Every E4M3 value is exactly a
bf16 value (3 mantissa bits within 7, exponents within range), which is how
the fp8 ragged_dot reuses the bf16 one.
"""

import numpy as np

from .bf16 import f32_to_bf16_bits
from .ragged import ragged_dot, trans_ragged_dot


def e4m3_to_f64(codes):
    """uint8 E4M3 codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (c & 7 == 7), np.nan, val)
    return np.where(s == 1, -val, val)


def e4m3_to_bf16_bits(codes):
    """uint8 E4M3 codes -> uint16 bf16 bits of the same value (exact)."""
    return f32_to_bf16_bits(e4m3_to_f64(codes).astype(np.float32))


def ragged_dot_fp8(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=True):
    """ragged_dot on E4M3 inputs: x uint8 [m, k], w uint8 [num_local, n, k] (trans_rhs) or [num_local, k, n].

    Returns float64 [L, n], exactly the bf16 ragged_dot of the same values.
    """
    return ragged_dot(e4m3_to_bf16_bits(x), e4m3_to_bf16_bits(w), group_sizes, group_offset, limit,
                      trans_rhs=trans_rhs)


def trans_ragged_dot_fp8(x, y, group_sizes, num_local=None, group_offset=None, limit=None):
    """trans_ragged_dot on E4M3 inputs: x uint8 [m, k], y uint8 [m, n] -> float64 [num_local, k, n].

    Exactly the bf16 trans_ragged_dot of the same values (the products are exact in float64).
    """
    return trans_ragged_dot(e4m3_to_bf16_bits(x), e4m3_to_bf16_bits(y), group_sizes, num_local, group_offset,
                            limit)

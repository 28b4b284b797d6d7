"""Pins of the unsort_bwd_rows oracle (what fixes it independently of itself).

MaxText PR #5760, commit on valid rows: grad = bf16(f32(g) * w) and the
float32 routing-weight row dot, over rows [0, limit).

* exact rational arithmetic: every product rounded to binary32 and then to
  bf16 by a rounding routine written here from the IEEE definition (not the
  oracle's bit trick), on random, tiny, huge and subnormal values;
* the float32 intermediate matters: inputs where rounding the exact product
  straight to bf16 gives a different result (double rounding) must follow
  the two-step rounding;
* special weights with known results: 1 (identity), -1 (sign flip), powers
  of two (exponent shift), 0 (signed zero);
* the dot: exact rational sums; y = e_c picks g[r, c]; y = g gives the sum of
  squares;
* the limit: clamping and that rows past it are absent.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.unsort as ounsort

# ---------------------------------------------------------------- exact rounding from the IEEE definition


def _round_binary(q, p, emin, emax):
    """Round the rational q to a binary format with p significand bits (normal exponents emin..emax),
    to nearest, ties to even; gradual underflow; overflow to +-inf (returned as a float)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * r


def _to_f32(q):
    return _round_binary(q, 24, -126, 127)


def _to_bf16(q):
    return _round_binary(q, 8, -126, 127)


def _frac(x):
    return Fraction(float(x))


def _bits_value(bits):
    return [float(v) for v in oracle.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))]


def _random_bf16(shape, rng, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return oracle.f32_to_bf16_bits(f)


@pytest.mark.parametrize("seed,scale,wscale", [(1, 1.0, 1.0), (2, 1e-20, 1e-20), (3, 1e18, 1e18),
                                               (4, 1e-38, 0.5), (5, 3.0, 1e-3)])
def test_grad_matches_exact_two_step_rounding(seed, scale, wscale):
    rng = np.random.default_rng(seed)
    rows, hidden = 6, 24
    g = _random_bf16((rows, hidden), rng, scale)
    y = _random_bf16((rows, hidden), rng)
    w = (rng.standard_normal(rows) * wscale).astype(np.float32)
    grad, _ = ounsort.unsort_bwd_rows(g, y, w)
    gv = _bits_value(g.ravel())
    for r in range(rows):
        for c in range(hidden):
            want = _to_bf16(_to_f32(_frac(gv[r * hidden + c]) * _frac(w[r])))
            got = _bits_value([grad[r, c]])[0]
            assert Fraction(got) == want, (r, c, gv[r * hidden + c], w[r])


def test_float32_intermediate_decides_double_rounding_cases():
    """Products whose float32 rounding lands exactly on a bf16 tie while the exact product does not:
    the two-step result (float32, then bf16) is what the page fixes, and it differs from rounding the
    exact product once for some of them."""
    rng = np.random.default_rng(7)
    n = 1 << 22
    gb = rng.integers(0x3F80, 0x4000, size=n).astype(np.uint16)           # bf16 in [1, 2)
    wf = (1.0 + rng.integers(1, 1 << 23, size=n) * 2.0 ** -23).astype(np.float32)
    p32 = oracle.bf16_bits_to_f32(gb) * wf                                # candidate filter only
    p64 = oracle.bf16_bits_to_f64(gb) * wf.astype(np.float64)             # exact (8 + 24 bits)
    cand = np.nonzero(((p32.view(np.uint32) & 0xFFFF) == 0x8000) & (p64 != p32.astype(np.float64)))[0]
    differ = []
    for i in cand:
        q = Fraction(float(p64[i]))
        two, one = _to_bf16(_to_f32(q)), _to_bf16(q)
        if two != one:
            differ.append((i, two))
    assert len(differ) >= 5
    idx = np.array([i for i, _ in differ])
    grad, _ = ounsort.unsort_bwd_rows(gb[idx][:, None], np.zeros((idx.size, 1), np.uint16), wf[idx])
    for k, (_, two) in enumerate(differ):
        assert Fraction(_bits_value([grad[k, 0]])[0]) == two


def test_special_weights():
    rng = np.random.default_rng(11)
    g = _random_bf16((5, 64), rng)
    g[0, :4] = [0x0000, 0x8000, 0x0001, 0x8001]     # +-0 and +-smallest subnormal
    y = _random_bf16((5, 64), rng)
    w = np.array([1.0, -1.0, 2.0 ** 10, 2.0 ** -3, 0.0], dtype=np.float32)
    grad, _ = ounsort.unsort_bwd_rows(g, y, w)
    assert np.array_equal(grad[0], g[0])                                   # x 1
    assert np.array_equal(grad[1], g[1] ^ 0x8000)                          # x -1
    e = ((g[2].astype(np.int32) >> 7) & 0xFF)
    normal = (e > 0) & (e + 10 < 255)
    assert np.array_equal(grad[2][normal], (g[2][normal].astype(np.int32) + (10 << 7)).astype(np.uint16))
    e3 = ((g[3].astype(np.int32) >> 7) & 0xFF)
    normal3 = e3 > 3
    assert np.array_equal(grad[3][normal3], (g[3][normal3].astype(np.int32) - (3 << 7)).astype(np.uint16))
    assert np.array_equal(grad[4], g[4] & 0x8000)                           # x +0 keeps g's sign on the zero


def test_dot_is_exact_sum_of_products():
    rng = np.random.default_rng(13)
    g = _random_bf16((4, 40), rng)
    y = _random_bf16((4, 40), rng)
    _, dot = ounsort.unsort_bwd_rows(g, y, np.ones(4, dtype=np.float32))
    gv = np.array(_bits_value(g.ravel())).reshape(g.shape)
    yv = np.array(_bits_value(y.ravel())).reshape(y.shape)
    for r in range(4):
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(gv[r], yv[r]))
        assert abs(Fraction(float(dot[r])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_dot_special_rows():
    rng = np.random.default_rng(17)
    g = _random_bf16((3, 32), rng)
    y = np.zeros_like(g)
    y[0, 5] = 0x3F80                                    # e_5
    y[1] = g[1]                                         # y = g
    _, dot = ounsort.unsort_bwd_rows(g, y, np.ones(3, dtype=np.float32))
    gv = np.array(_bits_value(g.ravel())).reshape(g.shape)
    assert dot[0] == gv[0, 5]
    assert dot[1] == pytest.approx(float((gv[1].astype(np.float64) ** 2).sum()), rel=1e-15) and dot[1] > 0
    assert dot[2] == 0.0


@pytest.mark.parametrize("limit,L", [(None, 9), (0, 0), (-5, 0), (4, 4), (9, 9), (100, 9)])
def test_limit_clamps_and_drops_rows(limit, L):
    rng = np.random.default_rng(19)
    g = _random_bf16((9, 16), rng)
    y = _random_bf16((9, 16), rng)
    w = rng.standard_normal(9).astype(np.float32)
    grad, dot = ounsort.unsort_bwd_rows(g, y, w, limit)
    full_grad, full_dot = ounsort.unsort_bwd_rows(g, y, w)
    assert grad.shape == (L, 16) and dot.shape == (L,)
    assert np.array_equal(grad, full_grad[:L]) and np.array_equal(dot, full_dot[:L])
    # each row depends only on its own weight
    w2 = w.copy()
    w2[L:] = 7.0
    g2, d2 = ounsort.unsort_bwd_rows(g, y, w2, limit)
    assert np.array_equal(g2, grad) and np.array_equal(d2, dot)

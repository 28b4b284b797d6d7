"""Pins for the GLU oracle and the bf16 rounding it ends with.

* RNE narrowing against torch's own float32 -> bfloat16 cast and hand-made ties;
* a special-value table whose results follow from IEEE-754 rules applied to
  the page's op sequence (negate, exp, + 1, divide, multiply), each entry
  with its reason;
* every one of the 65536 bf16 gate patterns x 64 random up values against the
  exact real-number silu(g) * u evaluated in float64: within 1 bf16 ulp
  everywhere the float32 sequence cannot overflow, and equal almost
  everywhere, while an op-by-op bf16-rounded variant (the alternative the
  MaxText page measures against) disagrees far more often;
* the backward against the float64 derivative of g * sigmoid(g) * u, whose
  formula is itself fixed by central differences, plus the -0 -> +0 rule.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits

NAN = "nan"


def bf(v):
    return int(f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])


def ulp_distance(a, b):
    """Distance between bf16 patterns on the ordered-integer line (+0 and -0 coincide)."""
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(oa - ob)


def is_nan_bits(b):
    b = np.asarray(b, dtype=np.int64)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


# ---------------------------------------------------------------- rounding


def test_rne_matches_torch_cast_on_random_patterns():
    rng = np.random.default_rng(0)
    pats = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = pats.view(np.float32)
    finite = np.isfinite(f)
    ours = f32_to_bf16_bits(f[finite])
    theirs = torch.from_numpy(f[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    nan_out = f32_to_bf16_bits(f[np.isnan(f)])
    assert np.all(is_nan_bits(nan_out))


@pytest.mark.parametrize("f32_bits,bf16_bits", [
    (0x3F808000, 0x3F80),  # tie, even below
    (0x3F818000, 0x3F82),  # tie, odd below -> up
    (0x3F808001, 0x3F81),  # just past the tie
    (0x00008000, 0x0000),  # denormal tie to even zero
    (0x00018000, 0x0002),  # denormal tie, odd below -> up
    (0x7F7FFFFF, 0x7F80),  # largest float32 rounds to +inf
    (0xFF7F8000, 0xFF80),  # tie at the top of the range rounds to -inf (even)
    (0x80000000, 0x8000),  # -0 stays -0
])
def test_rne_ties_and_edges(f32_bits, bf16_bits):
    v = np.array([f32_bits], dtype=np.uint32).view(np.float32)
    assert int(f32_to_bf16_bits(v)[0]) == bf16_bits


# ---------------------------------------------------------------- forward

# (gate bits, up bits, expected output bits or NAN, reason)
FWD_TABLE = [
    (0x0000, 0x3F80, 0x0000, "+0 / (1 + exp(-0)) = +0; +0 * 1 = +0"),
    (0x8000, 0x3F80, 0x8000, "-0 / 2 = -0; the forward keeps IEEE signs"),
    (0x0000, 0xBF80, 0x8000, "+0 * -1 = -0"),
    (0x7F80, 0x3F80, 0x7F80, "exp(-inf) = 0, den = 1, inf * 1 = inf"),
    (0x7F80, 0xC000, 0xFF80, "inf * -2 = -inf"),
    (0x7F80, 0x0000, NAN, "inf * 0 is NaN"),
    (0xFF80, 0x3F80, NAN, "exp(+inf) = inf, den = inf, -inf / inf is NaN"),
    (0x7FC0, 0x3F80, NAN, "NaN gate propagates"),
    (0x3F80, 0x7FC0, NAN, "NaN up propagates"),
    (0xC2C8, 0x3F80, 0x8000, "g = -100: exp(100) overflows float32, -100 / inf = -0"),
    (0x0002, 0x3F80, 0x0001, "denormal gate 2^-132: exp(-g) = 1, g / 2 = 2^-133, the smallest bf16 denormal"),
    (0x0002, 0x4040, 0x0003, "3 * 2^-133 is the bf16 denormal 3, exactly"),
    (0x0001, 0x4040, 0x0002, "3 * 2^-134 sits halfway between bf16 denormals 1 and 2: ties to even"),
    (0x0001, 0x3F80, 0x0000, "2^-134 is halfway between 0 and 2^-133: ties to even zero"),
    (0x3F80, 0x3F80, 0x3F3B, "silu(1) = 0.731058..., nearest bf16 1.0111011b * 2^-1"),
    (0xBF80, 0x3F80, 0xBE8A, "silu(-1) = -0.268941..., nearest bf16 -1.0001010b * 2^-2"),
    (0x4000, 0x4040, 0x40A9, "3 * silu(2) = 5.284782..., nearest bf16 1.0101001b * 2^2"),
]


@pytest.mark.parametrize("g,u,want,why", FWD_TABLE)
def test_glu_fwd_special_values(g, u, want, why):
    fused = np.array([[g, u]], dtype=np.uint16)
    got = int(oracle.glu_fwd(fused)[0, 0])
    if want == NAN:
        assert is_nan_bits(got), why
    else:
        assert got == want, (hex(got), why)


def exact_silu_times_up(g, u):
    """silu(g) * u in float64 (real-number reference)."""
    with np.errstate(over="ignore", invalid="ignore"):  # the sweeps include NaN and infinite gates
        g = g.astype(np.float64)
        u = u.astype(np.float64)
        return g * u / (1.0 + np.exp(-g))


def all_gate_sweep(reps, seed):
    gates = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(seed)
    ups = f32_to_bf16_bits(rng.standard_normal(reps).astype(np.float32))
    fused = np.empty((65536 * reps, 2), dtype=np.uint16)
    fused[:, 0] = np.repeat(gates, reps)
    fused[:, 1] = np.tile(ups, 65536)
    return fused


def test_glu_fwd_every_gate_against_exact_math():
    fused = all_gate_sweep(64, 1)
    got = oracle.glu_fwd(fused)[:, 0]
    g = bf16_bits_to_f32(fused[:, 0])
    u = bf16_bits_to_f32(fused[:, 1])
    exact = exact_silu_times_up(g, u)
    # where the float32 op sequence stays in range (exp(-g) finite, result normal or zero)
    ok = np.isfinite(g) & (g > -87.0) & np.isfinite(exact) & ((np.abs(exact) > 1e-37) | (exact == 0))
    with np.errstate(over="ignore"):  # exact values past the float32 range round to infinity, as the oracle's do
        want = f32_to_bf16_bits(exact[ok].astype(np.float32))
    d = ulp_distance(got[ok], want)
    assert d.max() <= 1
    assert np.mean(d == 0) > 0.999
    # negative control: rounding every intermediate to bf16 (the op-by-op alternative) disagrees often
    r = lambda a: bf16_bits_to_f32(f32_to_bf16_bits(a))
    with np.errstate(over="ignore", invalid="ignore", divide="ignore", under="ignore"):
        e = r(np.exp(-(g[ok].astype(np.float64))).astype(np.float32))
        opbyop = f32_to_bf16_bits(r(r(g[ok] / r(e + np.float32(1))) * u[ok]))
    assert np.mean(opbyop != got[ok]) > 0.005


def test_glu_fwd_limit_and_shape():
    rng = np.random.default_rng(2)
    fused = f32_to_bf16_bits(rng.standard_normal((20, 16)).astype(np.float32))
    full = oracle.glu_fwd(fused)
    assert full.shape == (20, 8)
    for limit, rows in [(None, 20), (0, 0), (7, 7), (20, 20), (99, 20), (-5, 0)]:
        got = oracle.glu_fwd(fused, limit)
        assert got.shape == (rows, 8)
        np.testing.assert_array_equal(got, full[:rows])
    # gate is the first half, up the second: swapping the halves changes the result
    swapped = np.concatenate([fused[:, 8:], fused[:, :8]], axis=1)
    assert np.any(oracle.glu_fwd(swapped) != full)


# ---------------------------------------------------------------- backward


def test_backward_formula_is_the_derivative():
    """Central differences of f(g) = g*sigmoid(g)*u in float64 against the closed form the oracle uses."""
    for g in np.linspace(-12, 12, 97):
        for u in (-1.7, 0.3, 2.0):
            f = lambda t: t * u / (1.0 + math.exp(-t))
            h = 1e-5
            fd = (f(g + h) - f(g - h)) / (2 * h)
            s = 1.0 / (1.0 + math.exp(-g))
            closed = u * s * (1.0 + g * (1.0 - s))
            assert abs(fd - closed) <= 1e-8 * max(1.0, abs(closed))


def test_glu_bwd_against_exact_derivative():
    rng = np.random.default_rng(3)
    n = 200000
    g = f32_to_bf16_bits((rng.standard_normal(n) * 4).astype(np.float32))
    u = f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    d = f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    fused = np.stack([g, u], axis=1)
    got = oracle.glu_bwd(fused, d[:, None])
    gf = bf16_bits_to_f32(g).astype(np.float64)
    uf = bf16_bits_to_f32(u).astype(np.float64)
    df = bf16_bits_to_f32(d).astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-gf))
    d_up = df * gf * s
    inner = 1.0 + gf * (1.0 - s)
    d_gate = df * uf * s * inner
    # d_up: a product chain, at most 1 bf16 ulp from the exact value
    want_up = f32_to_bf16_bits(d_up.astype(np.float32))
    want_up[want_up == 0x8000] = 0
    assert ulp_distance(got[:, 1], want_up).max() <= 1
    # d_gate: 1 + g(1 - s) cancels near silu's minimum (g ~ -1.278); compare where it is well conditioned
    cond = (np.abs(gf * (1.0 - s)) + 1.0) / np.abs(inner)
    ok = cond < 4.0
    want_gate = f32_to_bf16_bits(d_gate[ok].astype(np.float32))
    want_gate[want_gate == 0x8000] = 0
    dist = ulp_distance(got[ok, 0], want_gate)
    assert dist.max() <= 1
    assert np.mean(dist == 0) > 0.995
    assert ok.mean() > 0.9


def test_glu_bwd_maps_negative_zero_and_layout():
    # d = -0 makes both products -0 or +0; the output must hold no 0x8000
    g = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0xC2C8], dtype=np.uint16)
    u = np.array([0x3F80, 0x3F80, 0xBF80, 0x3F80, 0x3F80], dtype=np.uint16)
    d = np.array([0x8000, 0x8000, 0x3F80, 0x3F80, 0x3F80], dtype=np.uint16)
    fused = np.concatenate([g[None, :], u[None, :]], axis=1)
    out = oracle.glu_bwd(fused, d[None, :])
    assert out.shape == (1, 10)
    assert not np.any(out == 0x8000)
    # d_up of g = +0 with d = 1 is +0; d_gate of g = 0: d*u*0.5*(1 + 0) = -0.5 for u = -1
    assert out[0, 5 + 2] == 0x0000
    assert out[0, 2] == bf(-0.5)
    # g = -100: exp overflows, sigma = 0, silu = -0 -> d_up = -0 -> +0; d_gate = 0 * (1 + -100) = -0 -> +0
    assert out[0, 4] == 0x0000 and out[0, 9] == 0x0000


def test_glu_bwd_special_values():
    cases = [
        # (g, u, d, d_gate, d_up)
        (0x7F80, 0x3F80, 0x3F80, NAN, 0x7F80),  # sigma = 1: d_gate = 1*(1 + inf*0) -> NaN; d_up = inf
        (0xFF80, 0x3F80, 0x3F80, NAN, NAN),     # sigma = 0, silu = -inf/inf = NaN
        (0x7FC0, 0x3F80, 0x3F80, NAN, NAN),
        (0x3F80, 0x3F80, 0x3F80, bf(1 / (1 + math.exp(-1)) * (1 + 1 - 1 / (1 + math.exp(-1)))),
         bf(1 / (1 + math.exp(-1)))),
    ]
    for g, u, d, want_gate, want_up in cases:
        out = oracle.glu_bwd(np.array([[g, u]], dtype=np.uint16), np.array([[d]], dtype=np.uint16))
        for got, want in ((int(out[0, 0]), want_gate), (int(out[0, 1]), want_up)):
            if want == NAN:
                assert is_nan_bits(got)
            else:
                assert ulp_distance(got, want) <= 1


def test_glu_bwd_limit():
    rng = np.random.default_rng(4)
    fused = f32_to_bf16_bits(rng.standard_normal((12, 8)).astype(np.float32))
    d = f32_to_bf16_bits(rng.standard_normal((12, 4)).astype(np.float32))
    full = oracle.glu_bwd(fused, d)
    assert full.shape == (12, 8)
    np.testing.assert_array_equal(oracle.glu_bwd(fused, d, 5), full[:5])
    assert oracle.glu_bwd(fused, d, 0).shape == (0, 8)

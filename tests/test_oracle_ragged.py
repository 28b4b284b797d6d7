"""Pins for the ragged-dot oracle: each test checks it against something other than itself.

* brute force: pure-Python loops with their own per-row group search, on
  small-integer inputs where every sum is exact in float64;
* the SkyRL-tx page's own window algorithm (pad the first and last local
  groups, compute every row, mask), written out independently;
* dense closed forms (a single group is a plain matrix product; the local
  dW's sum to the window's dense x^T dy);
* exact finite differences of the linear maps <R, ragged_dot(x, w)> and
  <Z, trans_ragged_dot(x, y)>, which fix every transposition in the
  backward rules of the SkyRL-tx review.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_bits_to_f64, f32_to_bf16_bits


def int_bf16(rng, shape, lo=-3, hi=3):
    """bf16 bit patterns of small integers: products and sums stay exact in float64."""
    vals = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(vals)


def owner_of_row(r, gs):
    """Group owning row r by walking the sizes (negative sizes own nothing); None past the end."""
    start = 0
    for i, s in enumerate(gs):
        s = max(int(s), 0)
        if start <= r < start + s:
            return i
        start += s
    return None


def brute_ragged(x, w, gs, off, gl, limit, trans_rhs=False):
    m, k = len(x), len(x[0])
    n = len(w[0]) if trans_rhs else len(w[0][0])
    L = m if limit is None else min(max(limit, 0), m)
    G = len(gs)
    out = [[0.0] * n for _ in range(L)]
    if off < 0 or off + gl > G:
        return out
    for r in range(L):
        i = owner_of_row(r, gs)
        if i is None or not (off <= i < off + gl):
            continue
        j = i - off
        for c in range(n):
            acc = 0.0
            for t in range(k):
                wv = w[j][c][t] if trans_rhs else w[j][t][c]
                acc += x[r][t] * wv
            out[r][c] = acc
    return out


def brute_trans(x, y, gs, off, gl, limit):
    m, k = len(x), len(x[0])
    n = len(y[0])
    L = m if limit is None else min(max(limit, 0), m)
    out = [[[0.0] * n for _ in range(k)] for _ in range(gl)]
    if off < 0 or off + gl > len(gs):
        return out
    for r in range(L):
        i = owner_of_row(r, gs)
        if i is None or not (off <= i < off + gl):
            continue
        j = i - off
        for a in range(k):
            for c in range(n):
                out[j][a][c] += x[r][a] * y[r][c]
    return out


CASES = [
    # (gs, offset, num_local, limit)
    ([3, 0, 4, 2], None, 4, None),
    ([3, 0, 4, 2], 1, 2, None),
    ([3, 0, 4, 2], 0, 1, None),
    ([3, 0, 4, 2], 3, 1, None),
    ([3, 0, 4, 2], 1, 3, 6),
    ([3, 0, 4, 2], None, 4, 0),
    ([3, 0, 4, 2], None, 4, 5),
    ([0, 0, 0, 0], None, 4, None),
    ([5, -2, 3, 9], None, 4, None),   # negative size counts as 0; sum exceeds m
    ([5, -2, 3, 9], 2, 2, 100),       # limit above m clamps to m
    ([5, 2, 3, 1], 3, 2, None),       # window past the last group: empty
    ([5, 2, 3, 1], -1, 2, None),      # negative offset: empty
    ([1, 1, 1, 1], 0, 4, -3),         # negative limit: nothing valid
]


@pytest.mark.parametrize("gs,off,gl,limit", CASES)
@pytest.mark.parametrize("trans_rhs", [False, True])
def test_ragged_dot_matches_brute_force(gs, off, gl, limit, trans_rhs):
    rng = np.random.default_rng(len(gs) * 7 + gl + (0 if limit is None else limit))
    m, k, n = 10, 3, 4
    x = int_bf16(rng, (m, k))
    w = int_bf16(rng, (gl, n, k) if trans_rhs else (gl, k, n))
    got = oracle.ragged_dot(x, w, np.array(gs), group_offset=off, limit=limit, trans_rhs=trans_rhs)
    want = brute_ragged(bf16_bits_to_f64(x).tolist(), bf16_bits_to_f64(w).tolist(), gs,
                        0 if off is None else off, gl, limit, trans_rhs)
    assert got.shape == (len(want), n)
    np.testing.assert_array_equal(got, np.array(want, dtype=np.float64).reshape(got.shape))
    # masked rows are +0, not -0
    assert not np.any(np.signbit(got[got == 0]))


@pytest.mark.parametrize("gs,off,gl,limit", CASES)
def test_trans_ragged_dot_matches_brute_force(gs, off, gl, limit):
    rng = np.random.default_rng(11 + gl)
    m, k, n = 10, 3, 5
    x = int_bf16(rng, (m, k))
    y = int_bf16(rng, (m, n))
    got = oracle.trans_ragged_dot(x, y, np.array(gs), num_local=gl, group_offset=off, limit=limit)
    want = brute_trans(bf16_bits_to_f64(x).tolist(), bf16_bits_to_f64(y).tolist(), gs,
                       0 if off is None else off, gl, limit)
    np.testing.assert_array_equal(got, np.array(want))


def test_rows_subset_equals_full():
    rng = np.random.default_rng(3)
    m, k, n, G = 40, 8, 6, 5
    gs = np.array([7, 0, 12, 9, 5])
    x = int_bf16(rng, (m, k))
    w = int_bf16(rng, (3, k, n))
    full = oracle.ragged_dot(x, w, gs, group_offset=1, limit=30)
    rows = [0, 6, 7, 18, 19, 27, 28, 29]
    np.testing.assert_array_equal(oracle.ragged_dot(x, w, gs, group_offset=1, limit=30, rows=rows), full[rows])
    dw = oracle.trans_ragged_dot(x, int_bf16(rng, (m, n)), gs, num_local=3, group_offset=1, limit=30)
    assert dw.shape == (3, k, n)


def test_single_group_is_dense_matmul():
    """G = 1 reduces ragged_dot to a plain matrix product (checked with torch, not numpy)."""
    rng = np.random.default_rng(5)
    m, k, n = 33, 17, 9
    x = f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    w = f32_to_bf16_bits(rng.standard_normal((1, k, n)).astype(np.float32))
    got = oracle.ragged_dot(x, w, np.array([m]))
    want = torch.from_numpy(bf16_bits_to_f64(x)) @ torch.from_numpy(bf16_bits_to_f64(w[0]))
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-13, atol=1e-13)
    dy = f32_to_bf16_bits(rng.standard_normal((m, n)).astype(np.float32))
    dw = oracle.trans_ragged_dot(x, dy, np.array([m]))
    want_dw = torch.from_numpy(bf16_bits_to_f64(x)).T @ torch.from_numpy(bf16_bits_to_f64(dy))
    np.testing.assert_allclose(dw[0], want_dw.numpy(), rtol=1e-13, atol=1e-13)


def pages_window_algorithm(x, w_local, gs, off):
    """The SkyRL-tx review's fast_ragged_dot, restated: adjusted sizes, compute all rows, mask.

    The first local group absorbs every row before the shard and the last one
    every row after it; rows outside [shard_start, shard_end) are then zeroed.
    Evaluated with its own per-row loop (exact for small-integer inputs).
    """
    xs = bf16_bits_to_f64(x)
    ws = bf16_bits_to_f64(w_local)
    m = xs.shape[0]
    gl = ws.shape[0]
    cum = [0]
    for s in gs:
        cum.append(cum[-1] + int(s))
    shard_start, shard_end = cum[off], cum[off + gl]
    adjusted = [int(s) for s in gs[off : off + gl]]
    adjusted[0] += shard_start
    adjusted[-1] += m - shard_end
    result = np.zeros((m, ws.shape[2]))
    for r in range(m):
        j = owner_of_row(r, adjusted)
        result[r] = xs[r] @ ws[j]
    valid = np.array([(shard_start <= r < shard_end) for r in range(m)])
    return np.where(valid[:, None], result, 0.0)


@pytest.mark.parametrize("off,gl", [(0, 6), (0, 2), (2, 3), (5, 1), (1, 5), (3, 2)])
def test_window_matches_pages_algorithm_and_full_mask(off, gl):
    rng = np.random.default_rng(100 + off * 10 + gl)
    G, k, n = 6, 4, 3
    gs = np.array([4, 0, 6, 3, 0, 5])
    m = int(gs.sum())
    x = int_bf16(rng, (m, k))
    w_all = int_bf16(rng, (G, k, n))
    w_local = w_all[off : off + gl]
    got = oracle.ragged_dot(x, w_local, gs, group_offset=off)
    np.testing.assert_array_equal(got, pages_window_algorithm(x, w_local, gs, off))
    # the window result is the full-G result masked to [lo, hi)
    full = oracle.ragged_dot(x, w_all, gs)
    _, lo, hi, _ = oracle.boundaries(gs, m, off, gl)
    masked = full.copy()
    masked[:lo] = 0
    masked[hi:] = 0
    np.testing.assert_array_equal(got, masked)


def test_trans_rhs_is_transposed_weight():
    rng = np.random.default_rng(9)
    gs = np.array([5, 0, 7])
    x = int_bf16(rng, (12, 6))
    w = int_bf16(rng, (3, 4, 6))  # [g, n, k]
    a = oracle.ragged_dot(x, w, gs, trans_rhs=True)
    b = oracle.ragged_dot(x, np.ascontiguousarray(w.transpose(0, 2, 1)), gs)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("off,gl,limit", [(None, 5, None), (1, 3, None), (0, 5, 17), (2, 2, 9)])
def test_dw_sum_is_dense_window_product(off, gl, limit):
    """Sum over local groups of x_j^T dy_j equals x_win^T dy_win, the window's dense product."""
    rng = np.random.default_rng(21)
    gs = np.array([6, 0, 8, 3, 7])
    m, k, n = 26, 5, 4
    x = int_bf16(rng, (m, k))
    dy = int_bf16(rng, (m, n))
    dw = oracle.trans_ragged_dot(x, dy, gs, num_local=gl, group_offset=off, limit=limit)
    _, lo, hi, _ = oracle.boundaries(gs, m, off, gl, limit)
    dense = torch.from_numpy(bf16_bits_to_f64(x[lo:hi])).T @ torch.from_numpy(bf16_bits_to_f64(dy[lo:hi]))
    np.testing.assert_array_equal(dw.sum(axis=0), dense.numpy())
    lb, _, _, _ = oracle.boundaries(gs, m, off, gl, limit)
    for j in range(gl):
        if lb[j + 1] == lb[j]:
            assert np.all(dw[j] == 0) and not np.any(np.signbit(dw[j]))


def _perturbed(bits, idx, delta):
    v = bf16_bits_to_f64(bits).astype(np.float32)
    v[idx] += delta
    return f32_to_bf16_bits(v)


@pytest.mark.parametrize("off,limit", [(None, None), (1, None), (0, 9), (1, 11)])
def test_ragged_dot_vjp_by_exact_finite_differences(off, limit):
    """d<R, ragged_dot(x,w)>/dx = ragged_dot(R, w, trans_rhs) and /dw = trans_ragged_dot(x, R).

    The map is linear in each argument and every value is a small integer, so
    the central difference with step 1 is exact.
    """
    rng = np.random.default_rng(31 + (off or 0))
    G, m, k, n = 3, 13, 4, 3
    gs = np.array([4, 0, 8]) if off is None else np.array([2, 4, 0, 5])
    gl = 3
    x = int_bf16(rng, (m, k), -2, 2)
    w = int_bf16(rng, (gl, k, n), -2, 2)
    _, _, _, L = oracle.boundaries(gs, m, off, gl, limit)
    R = int_bf16(rng, (m, n), -2, 2)
    Rf = bf16_bits_to_f64(R)[:L]

    def f(xb, wb):
        return float(np.sum(Rf * oracle.ragged_dot(xb, wb, gs, group_offset=off, limit=limit)))

    dx_rule = np.zeros((m, k))
    # w is [g, k, n]; as a trans_rhs weight of R ([m, n]) it reads as [g, n_out=k, n].
    dx_rule[:L] = oracle.ragged_dot(R, w, gs, group_offset=off, limit=limit, trans_rhs=True)
    dw_rule = oracle.trans_ragged_dot(x, R, gs, num_local=gl, group_offset=off, limit=limit)
    for idx in np.ndindex(m, k):
        fd = (f(_perturbed(x, idx, 1.0), w) - f(_perturbed(x, idx, -1.0), w)) / 2
        assert fd == dx_rule[idx], idx
    for idx in np.ndindex(gl, k, n):
        fd = (f(x, _perturbed(w, idx, 1.0)) - f(x, _perturbed(w, idx, -1.0))) / 2
        assert fd == dw_rule[idx], idx


def test_trans_ragged_dot_vjp_by_exact_finite_differences():
    """For z = trans_ragged_dot(x, y): dx = ragged_dot(y, dz, trans_rhs) and dy = ragged_dot(x, dz).

    This is the corrected rule of the SkyRL-tx review (the page's first version
    used trans_ragged_dot for dy, which cannot even take dz's shape).
    """
    rng = np.random.default_rng(41)
    gs = np.array([3, 0, 5, 2])
    G, m, k, n = 4, 10, 3, 4
    x = int_bf16(rng, (m, k), -2, 2)
    y = int_bf16(rng, (m, n), -2, 2)
    Z = int_bf16(rng, (G, k, n), -2, 2)
    Zf = bf16_bits_to_f64(Z)

    def f(xb, yb):
        return float(np.sum(Zf * oracle.trans_ragged_dot(xb, yb, gs)))

    # dz has layout [g, k, n]; as the trans_rhs weight of y ([m, n]) it is [g, n_out=k, n].
    dx_rule = oracle.ragged_dot(y, Z, gs, trans_rhs=True)
    dy_rule = oracle.ragged_dot(x, Z, gs)
    for idx in np.ndindex(m, k):
        fd = (f(_perturbed(x, idx, 1.0), y) - f(_perturbed(x, idx, -1.0), y)) / 2
        assert fd == dx_rule[idx], idx
    for idx in np.ndindex(m, n):
        fd = (f(x, _perturbed(y, idx, 1.0)) - f(x, _perturbed(y, idx, -1.0))) / 2
        assert fd == dy_rule[idx], idx


def test_boundaries_invariants_over_page_limits():
    """The limit sweeps the MaxText page checks, on a scaled-down buffer: boundaries stay ordered and clamped."""
    rng = np.random.default_rng(7)
    gs = rng.multinomial(1262, np.full(256, 1 / 256))
    m = 2253
    for limit in [0, 1, 10, 1259, 1262, 2253, 5000, -4]:
        lb, lo, hi, L = oracle.boundaries(gs, m, 96, 32, limit)
        assert 0 <= lo <= hi <= L <= m
        assert np.all(np.diff(lb) >= 0)
        cum = np.concatenate([[0], np.cumsum(gs)])
        assert lo == min(cum[96], L) and hi == min(cum[128], L)

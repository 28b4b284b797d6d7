"""Pins of the fp8 (E4M3) oracle.

* The decode of all 256 codes against torch's own float8_e4m3fn conversion
  (an independent implementation) and against values the format fixes.
* The fp8 ragged_dot against a brute-force triple loop over the decoded
  values, and (g = 1) against a dense float64 matmul of torch-decoded values.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ofp8.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x7E, 448.0), (0x01, 2.0 ** -9),
                                        (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0xB8, -1.0), (0xFE, -448.0),
                                        (0x3C, 1.5), (0x30, 0.5)])
def test_format_values(code, value):
    assert ofp8.e4m3_to_f64(np.array([code], dtype=np.uint8))[0] == value


def test_nan_codes_and_negative_zero():
    v = ofp8.e4m3_to_f64(np.array([0x7F, 0xFF, 0x80], dtype=np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])


def test_every_code_is_exactly_a_bf16_value():
    codes = np.arange(256, dtype=np.uint8)
    vals = ofp8.e4m3_to_f64(codes)
    back = oracle.bf16_bits_to_f64(ofp8.e4m3_to_bf16_bits(codes))
    fin = ~np.isnan(vals)
    assert np.array_equal(back[fin], vals[fin])


def _codes(shape, rng):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN inputs
    return c


@pytest.mark.parametrize("trans_rhs", [True, False])
def test_ragged_dot_fp8_brute_force(trans_rhs):
    rng = np.random.default_rng(5)
    gs = np.array([3, 0, 4, 2], dtype=np.int32)
    m, k, n = 11, 6, 5
    x = _codes((m, k), rng)
    w = _codes((4, n, k) if trans_rhs else (4, k, n), rng)
    got = ofp8.ragged_dot_fp8(x, w, gs, limit=10, trans_rhs=trans_rhs)
    xv, wv = ofp8.e4m3_to_f64(x), ofp8.e4m3_to_f64(w)
    lb = np.concatenate([[0], np.cumsum(gs)])
    for r in range(10):
        for c in range(n):
            j = [g for g in range(4) if lb[g] <= r < lb[g + 1]]
            want = 0.0
            if j:
                for t in range(k):
                    want += xv[r, t] * (wv[j[0], c, t] if trans_rhs else wv[j[0], t, c])
            assert got[r, c] == want


def test_single_group_is_dense_matmul():
    rng = np.random.default_rng(6)
    x = _codes((40, 64), rng)
    w = _codes((1, 24, 64), rng)
    got = ofp8.ragged_dot_fp8(x, w, np.array([40], dtype=np.int32))
    xt = torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float64)
    wt = torch.from_numpy(w[0]).view(torch.float8_e4m3fn).to(torch.float64)
    assert np.allclose(got, (xt @ wt.T).numpy(), rtol=1e-15, atol=0)


def test_trans_ragged_dot_fp8_brute_force():
    """dw[j][a, c] = sum over group j's rows of x[r, a] * y[r, c], with torch's own E4M3 decode; an empty
    group gives +0; rows past the limit and outside the window contribute nothing."""
    rng = np.random.default_rng(7)
    gs = np.array([4, 0, 3, 5], dtype=np.int32)
    m, k, n = 13, 5, 6
    x = _codes((m, k), rng)
    y = _codes((m, n), rng)
    got = ofp8.trans_ragged_dot_fp8(x, y, gs, num_local=3, group_offset=1, limit=10)
    xv = torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    yv = torch.from_numpy(y).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    lb = np.minimum(np.concatenate([[0], np.cumsum(gs)]), 10)
    assert got.shape == (3, k, n)
    for j in range(3):
        want = np.zeros((k, n))
        for r in range(lb[1 + j], lb[2 + j]):
            for a in range(k):
                for c in range(n):
                    want[a, c] += xv[r, a] * yv[r, c]
        assert np.array_equal(got[j], want), j
    assert np.all(got[0] == 0) and not np.signbit(got[0]).any()

"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of an oracle function (on the CPU,
by monkeypatching) and runs the pin tests that should notice it; the case
passes only if at least one of those pins fails.
"""

import numpy as np
import pytest

import oracle
import oracle.glu as oglu
import oracle.ragged as orag
from oracle.bf16 import bf16_bits_to_f32, bf16_bits_to_f64, f32_to_bf16_bits

from tests import test_oracle_glu as pg
from tests import test_oracle_ragged as pr
from tests import test_oracle_unsort as pu
import oracle.unsort as ouns


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    except (ValueError, IndexError):
        return True
    return False


def _ragged_pins():
    yield pr.test_ragged_dot_matches_brute_force, ([3, 0, 4, 2], 1, 2, None, False)
    yield pr.test_ragged_dot_matches_brute_force, ([3, 0, 4, 2], 1, 3, 6, True)
    yield pr.test_ragged_dot_matches_brute_force, ([5, -2, 3, 9], None, 4, None, False)
    yield pr.test_ragged_dot_matches_brute_force, ([1, 1, 1, 1], 0, 4, -3, False)
    yield pr.test_window_matches_pages_algorithm_and_full_mask, (2, 3)
    yield pr.test_trans_rhs_is_transposed_weight, ()
    yield pr.test_ragged_dot_vjp_by_exact_finite_differences, (1, 11)
    yield pr.test_trans_ragged_dot_vjp_by_exact_finite_differences, ()
    yield pr.test_trans_ragged_dot_matches_brute_force, ([3, 0, 4, 2], 1, 3, 6)
    yield pr.test_dw_sum_is_dense_window_product, (1, 3, None)
    yield pr.test_single_group_is_dense_matmul, ()


def _caught(pins):
    return any(_fails(fn, *args) for fn, args in pins)


# ---------------------------------------------------------------- ragged mutants


def _window_off_by_one(group_sizes, m, group_offset=None, num_local=None, limit=None):
    lb, lo, hi, L = _orig_boundaries(group_sizes, m, group_offset, num_local, limit)
    if group_offset:
        lb2, _, _, _ = _orig_boundaries(group_sizes, m, group_offset + 1 if group_offset + 1 + (num_local or 0) <= len(group_sizes) else group_offset, num_local, limit)
        lb = lb2
    return lb, int(lb[0]), int(lb[-1]), L


def _limit_ignored(group_sizes, m, group_offset=None, num_local=None, limit=None):
    return _orig_boundaries(group_sizes, m, group_offset, num_local, None)


def _negative_sizes_kept(group_sizes, m, group_offset=None, num_local=None, limit=None):
    gs = np.asarray(group_sizes, dtype=np.int64)
    G = gs.size
    L = m if limit is None else min(max(int(limit), 0), int(m))
    off = 0 if group_offset is None else int(group_offset)
    gl = G if num_local is None else int(num_local)
    if off < 0 or off + gl > G:
        return np.zeros(gl + 1, np.int64), 0, 0, L
    cum = np.concatenate([[0], np.cumsum(gs)])  # mistake: no clamp of negative sizes
    b = np.clip(cum, 0, L)
    lb = b[off : off + gl + 1]
    return lb, int(lb[0]), int(lb[-1]), L


_orig_boundaries = orag.boundaries


@pytest.mark.parametrize("mutant", [_window_off_by_one, _limit_ignored, _negative_sizes_kept])
def test_boundary_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(orag, "boundaries", mutant)
    monkeypatch.setattr(oracle, "boundaries", mutant)
    assert _caught(_ragged_pins())


def test_untransposed_rhs_is_caught(monkeypatch):
    orig = orag.ragged_dot

    def mutant(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False, rows=None):
        if trans_rhs:  # mistake: reinterpret the [g, n, k] memory as [g, k, n]
            w = np.ascontiguousarray(w).reshape(w.shape[0], w.shape[2], w.shape[1])
            return orig(x, w, group_sizes, group_offset, limit, False, rows)
        return orig(x, w, group_sizes, group_offset, limit, trans_rhs, rows)

    monkeypatch.setattr(oracle, "ragged_dot", mutant)
    assert _caught(_ragged_pins())


def test_shifted_group_weight_is_caught(monkeypatch):
    orig = orag.ragged_dot

    def mutant(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False, rows=None):
        w = np.roll(np.asarray(w), 1, axis=0)  # mistake: group j uses w[j-1]
        return orig(x, w, group_sizes, group_offset, limit, trans_rhs, rows)

    monkeypatch.setattr(oracle, "ragged_dot", mutant)
    assert _caught(_ragged_pins())


def test_trans_with_swapped_operands_is_caught(monkeypatch):
    def mutant(x, y, group_sizes, num_local=None, group_offset=None, limit=None, k_index=None):
        x = np.asarray(x, np.uint16)
        y = np.asarray(y, np.uint16)
        G = np.asarray(group_sizes).size
        gl = G if num_local is None else num_local
        lb, _, _, _ = orag.boundaries(group_sizes, x.shape[0], group_offset, gl, limit)
        out = np.zeros((gl, x.shape[1], y.shape[1]))
        for j in range(gl):
            s, e = int(lb[j]), int(lb[j + 1])
            # mistake: a row-reversed y (the rows of x and y no longer pair up)
            out[j] = bf16_bits_to_f64(x[s:e]).T @ bf16_bits_to_f64(y[s:e][::-1])
        return out

    monkeypatch.setattr(oracle, "trans_ragged_dot", mutant)
    assert _caught(_ragged_pins())


# ---------------------------------------------------------------- GLU mutants


def _glu_pins():
    yield pg.test_glu_fwd_every_gate_against_exact_math, ()
    for row in pg.FWD_TABLE:
        yield pg.test_glu_fwd_special_values, row
    yield pg.test_glu_fwd_limit_and_shape, ()
    yield pg.test_glu_bwd_against_exact_derivative, ()
    yield pg.test_glu_bwd_maps_negative_zero_and_layout, ()
    yield pg.test_glu_bwd_special_values, ()
    yield pg.test_glu_bwd_limit, ()


def test_op_by_op_rounding_is_caught(monkeypatch):
    def mutant(fused, limit=None):
        fused = np.asarray(fused, np.uint16)
        h = fused.shape[1] // 2
        L = fused.shape[0] if limit is None else min(max(limit, 0), fused.shape[0])
        r = lambda a: bf16_bits_to_f32(f32_to_bf16_bits(a))
        g = bf16_bits_to_f32(fused[:L, :h])
        u = bf16_bits_to_f32(fused[:L, h:])
        with np.errstate(all="ignore"):
            e = r(np.exp(-(g.astype(np.float64))).astype(np.float32))
            return f32_to_bf16_bits(r(r(g / r(e + np.float32(1))) * u))

    monkeypatch.setattr(oracle, "glu_fwd", mutant)
    assert _caught(_glu_pins())


def test_sigmoid_instead_of_silu_is_caught(monkeypatch):
    def mutant(fused, limit=None):
        fused = np.asarray(fused, np.uint16)
        h = fused.shape[1] // 2
        g = bf16_bits_to_f32(fused[:, :h])
        u = bf16_bits_to_f32(fused[:, h:])
        with np.errstate(all="ignore"):
            e = np.exp(-(g.astype(np.float64))).astype(np.float32)
            return f32_to_bf16_bits((np.float32(1) / (e + np.float32(1))) * u)  # mistake: drops the gate factor

    monkeypatch.setattr(oracle, "glu_fwd", mutant)
    assert _caught(_glu_pins())


def test_backward_without_inner_term_is_caught(monkeypatch):
    def mutant(fused, d_out, limit=None):
        fused = np.asarray(fused, np.uint16)
        h = fused.shape[1] // 2
        L = fused.shape[0] if limit is None else min(max(limit, 0), fused.shape[0])
        g = bf16_bits_to_f32(fused[:L, :h])
        u = bf16_bits_to_f32(fused[:L, h:])
        d = bf16_bits_to_f32(np.asarray(d_out, np.uint16)[:L])
        with np.errstate(all="ignore"):
            den = np.exp(-(g.astype(np.float64))).astype(np.float32) + np.float32(1)
            sig = np.float32(1) / den
            d_up = d * (g / den)
            d_gate = (d * u) * sig  # mistake: drops (1 + g (1 - s))
        out = np.concatenate([f32_to_bf16_bits(d_gate), f32_to_bf16_bits(d_up)], axis=1)
        out[out == 0x8000] = 0
        return out

    monkeypatch.setattr(oracle, "glu_bwd", mutant)
    assert _caught(_glu_pins())


def test_missing_negative_zero_map_is_caught(monkeypatch):
    orig = oglu.glu_bwd

    def mutant(fused, d_out, limit=None):
        out = orig(fused, d_out, limit)
        # undo the map where the float32 product was -0 (recompute the signs of zero results)
        fused = np.asarray(fused, np.uint16)
        h = fused.shape[1] // 2
        L = out.shape[0]
        g = bf16_bits_to_f32(fused[:L, :h])
        d = bf16_bits_to_f32(np.asarray(d_out, np.uint16)[:L])
        with np.errstate(all="ignore"):
            s = g / (np.exp(-(g.astype(np.float64))).astype(np.float32) + np.float32(1))
            neg_zero = (out[:, h:] == 0) & np.signbit(d * s)
        out[:, h:][neg_zero] = 0x8000
        return out

    monkeypatch.setattr(oracle, "glu_bwd", mutant)
    assert _caught(_glu_pins())


# ---------------------------------------------------------------- unsort_bwd_rows mutants


def _unsort_pins():
    for args in ((1, 1.0, 1.0), (4, 1e-38, 0.5)):
        yield pu.test_grad_matches_exact_two_step_rounding, args
    yield pu.test_float32_intermediate_decides_double_rounding_cases, ()
    yield pu.test_special_weights, ()
    yield pu.test_dot_is_exact_sum_of_products, ()
    yield pu.test_dot_special_rows, ()
    for args in ((4, 4), (-5, 0), (100, 9)):
        yield pu.test_limit_clamps_and_drops_rows, args


def _unsort_with(grad_fn=None, dot_fn=None, limit_fn=None):
    def mutant(g, y, w, limit=None):
        g = np.asarray(g, dtype=np.uint16)
        y = np.asarray(y, dtype=np.uint16)
        w = np.asarray(w, dtype=np.float32)
        rows = g.shape[0]
        L = limit_fn(limit, rows) if limit_fn else (rows if limit is None else min(max(int(limit), 0), rows))
        gd = grad_fn(g[:L], w[:L]) if grad_fn else f32_to_bf16_bits(bf16_bits_to_f32(g[:L]) * w[:L, None])
        dt = dot_fn(g[:L], y[:L]) if dot_fn else (bf16_bits_to_f64(g[:L]) * bf16_bits_to_f64(y[:L])).sum(axis=1)
        return gd, dt
    return mutant


def _one_rounding(g, w):
    """the product rounded once from its exact value (float64) instead of through float32"""
    p = bf16_bits_to_f64(g) * w.astype(np.float64)[:, None]
    b = p.view(np.uint64)
    keep = (b >> 45) & 1
    r = (b + ((1 << 44) - 1) + keep) >> 45          # RNE to 8 significand bits, then back to float32 layout
    f = ((r << 45).view(np.float64)).astype(np.float32)
    return f32_to_bf16_bits(f)


def _shifted_weight(g, w):
    return f32_to_bf16_bits(bf16_bits_to_f32(g) * np.roll(w, 1)[:, None])


@pytest.mark.parametrize("mutant", [
    _unsort_with(grad_fn=_one_rounding),
    _unsort_with(grad_fn=_shifted_weight),
    _unsort_with(dot_fn=lambda g, y: (bf16_bits_to_f64(g) * bf16_bits_to_f64(g)).sum(axis=1)),
    _unsort_with(dot_fn=lambda g, y: (bf16_bits_to_f64(g) * bf16_bits_to_f64(y))[:, 1:].sum(axis=1)),
    _unsort_with(limit_fn=lambda limit, rows: rows),
    _unsort_with(limit_fn=lambda limit, rows: rows if limit is None else min(max(int(limit), 0) + 1, rows)),
], ids=["one-rounding", "shifted-weight", "dot-g-squared", "dot-drops-column", "limit-ignored", "limit-off-by-one"])
def test_unsort_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(ouns, "unsort_bwd_rows", mutant)
    assert _caught(_unsort_pins())

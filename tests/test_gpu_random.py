"""Seeded random cases of the three GEMMs against the oracle, every element.

Each case draws the group count, the sizes (Dirichlet shares, some groups
empty, sums below, at or past m), k and n (multiples of 8, across the tile
edges), an optional window and an optional limit (negative, inside, past m),
fills rows past the valid ones with NaN, and checks ragged_dot in both forms
and trans_ragged_dot (with and without the row-split workspace) against the
float64 oracle, plus the row contract (+0 outside the window below the limit,
rows at or past the limit untouched) and bf16 = RNE(float32).
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd
from expert_ffn_ragged_amd.workloads import bits, bf16_normal
from tests.gpu_util import (assert_bf16_is_rne_of_f32, assert_gemm_close, is_pos_zero, is_sentinel, say,
                            sentinel)

pytestmark = pytest.mark.gpu

DEV = "cuda"
CASES = 24


def dev_i32(v):
    return None if v is None else torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.integers(1, 41))
    total = int(rng.integers(0, 3000))
    shares = rng.dirichlet(np.full(G, float(rng.choice([0.2, 1.0, 5.0]))))
    sizes = rng.multinomial(total, shares).astype(np.int32)
    sizes[rng.random(G) < 0.15] = 0
    m = max(1, int(sizes.sum()) + int(rng.integers(-200, 300)))
    k = int(8 * rng.integers(1, 66))
    n = int(8 * rng.integers(1, 66))
    off = gl = None
    if G > 1 and rng.random() < 0.4:
        off = int(rng.integers(0, G))
        gl = int(rng.integers(1, G - off + 1))
    limit = None
    if rng.random() < 0.5:
        limit = int(rng.choice([-5, rng.integers(0, m + 1), m + 17]))
    return dict(G=G, sizes=sizes, m=m, k=k, n=n, off=off, gl=gl, limit=limit, seed=seed)


@pytest.mark.parametrize("seed", range(CASES))
def test_random_case(seed):
    c = draw(seed)
    G, sizes, m, k, n, off, limit = c["G"], c["sizes"], c["m"], c["k"], c["n"], c["off"], c["limit"]
    gl = G if c["gl"] is None else c["gl"]
    say(f"random case {seed}: G={G} m={m} k={k} n={n} off={off} gl={gl} limit={limit} sizes={sizes.tolist()}")
    lb, lo, hi, L = oracle.boundaries(sizes, m, off, gl, limit)
    valid = int(lb[-1])
    gs = torch.tensor(sizes, dtype=torch.int32, device=DEV)
    x = bf16_normal((m, k), 1.0, 10 * seed + 1, "cpu", nan_rows_from=max(valid, hi)).to(DEV)
    offt, limt = dev_i32(off), dev_i32(limit)
    outside = np.ones(L, dtype=bool)
    outside[lo:hi] = False
    outside = torch.from_numpy(outside).to(DEV)
    for trans_rhs in (False, True):
        w = bf16_normal((gl, n, k) if trans_rhs else (gl, k, n), 0.05, 10 * seed + 2, "cpu").to(DEV)
        o32 = sentinel((m, n), torch.float32)
        o16 = sentinel((m, n), torch.bfloat16)
        rd.ragged_dot(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o32)
        rd.ragged_dot(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o16)
        torch.cuda.synchronize()
        what = f"case {seed} trans_rhs={trans_rhs}"
        ref = oracle.ragged_dot(bits(x), bits(w), sizes, off, limit, trans_rhs)
        assert_gemm_close(o32[:L].cpu().numpy(), ref, what)
        assert bool(is_pos_zero(o32[:L][outside]).all()) and bool(is_pos_zero(o16[:L][outside]).all()), what
        assert bool(is_sentinel(o32[L:]).all()) and bool(is_sentinel(o16[L:]).all()), what + ": rows >= L written"
        assert_bf16_is_rne_of_f32(o16[:L], o32[:L], what)
    dy = bf16_normal((m, n), 1.0, 10 * seed + 3, "cpu", nan_rows_from=max(valid, hi)).to(DEV)
    ref = oracle.trans_ragged_dot(bits(x), bits(dy), sizes, gl, off, limit)
    for split in (True, False):
        d32 = sentinel((gl, k, n), torch.float32)
        d16 = sentinel((gl, k, n), torch.bfloat16)
        rd.trans_ragged_dot(x, dy, gs, gl, offt, limt, out=d32, row_split=split)
        rd.trans_ragged_dot(x, dy, gs, gl, offt, limt, out=d16, row_split=split)
        torch.cuda.synchronize()
        what = f"case {seed} dW split={split}"
        assert_gemm_close(d32.cpu().numpy(), ref, what)
        assert_bf16_is_rne_of_f32(d16, d32, what)


CASES_FP8 = 12


def fp8_normal(shape, std, seed, nan_rows_from=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = (torch.randn(shape, generator=g, device=DEV) * std).to(torch.float8_e4m3fn)
    if nan_rows_from is not None:
        t.view(torch.uint8)[nan_rows_from:] = 0x7F  # E4M3 NaN: rows that must not be read
    return t


def codes(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


@pytest.mark.parametrize("seed", range(CASES_FP8))
def test_random_fp8_case(seed):
    """The same draws with fp8 (E4M3) operands: both ragged_dot forms (k a multiple of 128, n of 16) and
    trans_ragged_dot (k and n multiples of 16, with and without the row split) against the oracle on the
    same values, the row contract, and bf16 = RNE(float32)."""
    c = draw(500 + seed)
    G, sizes, m, off, limit = c["G"], c["sizes"], c["m"], c["off"], c["limit"]
    gl = G if c["gl"] is None else c["gl"]
    rng = np.random.default_rng(2000 + seed)
    k, n = int(128 * rng.integers(1, 7)), int(16 * rng.integers(1, 33))
    say(f"random fp8 case {seed}: G={G} m={m} k={k} n={n} off={off} gl={gl} limit={limit} sizes={sizes.tolist()}")
    lb, lo, hi, L = oracle.boundaries(sizes, m, off, gl, limit)
    valid = int(lb[-1])
    gs = torch.tensor(sizes, dtype=torch.int32, device=DEV)
    x = fp8_normal((m, k), 1.0, 10 * seed + 5, max(valid, hi))
    offt, limt = dev_i32(off), dev_i32(limit)
    outside = np.ones(L, dtype=bool)
    outside[lo:hi] = False
    outside = torch.from_numpy(outside).to(DEV)
    for trans_rhs in (False, True):
        w = fp8_normal((gl, n, k) if trans_rhs else (gl, k, n), 0.5, 10 * seed + 6)
        o32 = sentinel((m, n), torch.float32)
        o16 = sentinel((m, n), torch.bfloat16)
        rd.ragged_dot_fp8(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o32)
        rd.ragged_dot_fp8(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o16)
        torch.cuda.synchronize()
        what = f"fp8 case {seed} trans_rhs={trans_rhs}"
        ref = oracle.ragged_dot_fp8(codes(x), codes(w), sizes, off, limit, trans_rhs=trans_rhs)
        assert_gemm_close(o32[:L].cpu().numpy(), ref, what)
        assert bool(is_pos_zero(o32[:L][outside]).all()) and bool(is_pos_zero(o16[:L][outside]).all()), what
        assert bool(is_sentinel(o32[L:]).all()) and bool(is_sentinel(o16[L:]).all()), what + ": rows >= L written"
        assert_bf16_is_rne_of_f32(o16[:L], o32[:L], what)
    kt, nt = int(16 * rng.integers(1, 41)), int(16 * rng.integers(1, 41))
    xt = fp8_normal((m, kt), 1.0, 10 * seed + 7, max(valid, hi))
    dy = fp8_normal((m, nt), 1.0, 10 * seed + 8, max(valid, hi))
    ref = oracle.trans_ragged_dot_fp8(codes(xt), codes(dy), sizes, gl, off, limit)
    for split in (True, False):
        d32 = sentinel((gl, kt, nt), torch.float32)
        d16 = sentinel((gl, kt, nt), torch.bfloat16)
        rd.trans_ragged_dot_fp8(xt, dy, gs, gl, offt, limt, out=d32, row_split=split)
        rd.trans_ragged_dot_fp8(xt, dy, gs, gl, offt, limt, out=d16, row_split=split)
        torch.cuda.synchronize()
        what = f"fp8 case {seed} dW k={kt} n={nt} split={split}"
        assert_gemm_close(d32.cpu().numpy(), ref, what)
        assert_bf16_is_rne_of_f32(d16, d32, what)

"""Every grouped-GEMM tile shape against the oracle.

The host picks a tile shape from m, k, n and num_local; the tuning hook
(rd_tune_set, ``rd.tuning``) forces one.  Each shape runs the
three GEMMs on one ragged case (groups against every tile edge, an empty
group, a window and a limit with NaN rows past it) and must meet the same
bar as the default choice: float32 output within the GEMM tolerance of the
oracle, bf16 output the RNE of the float32 one, rows below the limit outside
the window +0, rows past it untouched, dW of an empty group +0.
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd
from expert_ffn_ragged_amd.workloads import bf16_normal, bits
from tests.gpu_util import assert_bf16_is_rne_of_f32, assert_gemm_close, is_pos_zero, is_sentinel, say, sentinel

pytestmark = pytest.mark.gpu

DEV = "cuda"
TILE_SHAPES = list(range(19))  # rd.tile_count() shapes; a test below checks the count

GS = np.array([37, 0, 300, 129, 1, 200, 64], dtype=np.int32)
M, K, N = int(GS.sum()) + 23, 320, 576
OFF, GL = 1, 5
LIMIT = int(GS.sum()) - 90


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


@pytest.fixture(scope="module")
def case():
    x = bf16_normal((M, K), 1.0, 301, "cpu", nan_rows_from=LIMIT).to(DEV)
    w = bf16_normal((GL, K, N), 0.05, 302, "cpu").to(DEV)
    wt = bf16_normal((GL, N, K), 0.05, 303, "cpu").to(DEV)
    dy = bf16_normal((M, N), 1.0, 304, "cpu", nan_rows_from=LIMIT).to(DEV)
    return x, w, wt, dy


@pytest.mark.parametrize("tile", TILE_SHAPES)
def test_tile_shape_forward_forms(case, tile):
    say(f"tile {tile} forward and trans_rhs")
    x, w, wt, _ = case
    gs = torch.from_numpy(GS).to(DEV)
    lb, lo, hi, L = oracle.boundaries(GS, M, OFF, GL, LIMIT)
    for trans_rhs, wgt in ((False, w), (True, wt)):
        o32 = sentinel((M, N), torch.float32)
        o16 = sentinel((M, N), torch.bfloat16)
        with rd.tuning(fwd_tile=tile, decode=False):
            rd.ragged_dot(x, wgt, gs, dev_i32(OFF), dev_i32(LIMIT), trans_rhs=trans_rhs, out=o32)
            rd.ragged_dot(x, wgt, gs, dev_i32(OFF), dev_i32(LIMIT), trans_rhs=trans_rhs, out=o16)
        torch.cuda.synchronize()
        what = f"tile {tile} trans_rhs={trans_rhs}"
        ref = oracle.ragged_dot(bits(x), bits(wgt), GS, OFF, LIMIT, trans_rhs)
        assert_gemm_close(o32[:L].cpu().numpy(), ref, what)
        assert_bf16_is_rne_of_f32(o16[:L], o32[:L], what)
        assert bool(is_pos_zero(o32[:lo]).all()) and bool(is_pos_zero(o32[hi:L]).all()), what
        assert bool(is_sentinel(o32[L:]).all()) and bool(is_sentinel(o16[L:]).all()), what


@pytest.mark.parametrize("tile", TILE_SHAPES)
def test_tile_shape_trans_ragged_dot(case, tile):
    say(f"tile {tile} trans_ragged_dot")
    x, _, _, dy = case
    gs = torch.from_numpy(GS).to(DEV)
    d32 = sentinel((GL, K, N), torch.float32)
    d16 = sentinel((GL, K, N), torch.bfloat16)
    with rd.tuning(trans_tile=tile):
        rd.trans_ragged_dot(x, dy, gs, GL, dev_i32(OFF), dev_i32(LIMIT), out=d32)
        rd.trans_ragged_dot(x, dy, gs, GL, dev_i32(OFF), dev_i32(LIMIT), out=d16)
    torch.cuda.synchronize()
    what = f"tile {tile} dW"
    ref = oracle.trans_ragged_dot(bits(x), bits(dy), GS, GL, OFF, LIMIT)
    assert_gemm_close(d32.cpu().numpy(), ref, what)
    assert_bf16_is_rne_of_f32(d16, d32, what)
    assert bool(is_pos_zero(d32[0]).all()) and bool(is_pos_zero(d16[0]).all()), what + ": empty group"


def test_every_tile_shape_is_covered():
    assert rd.tile_count() == len(TILE_SHAPES)

"""GPU parity at the edges of the declared range, against the oracle, every element.

* RD_MAX_GROUPS = 1024 groups, all local: the device schedule's last-slot
  branches (a block of 256 threads scans 4 groups per thread, so 1024 groups
  fill it exactly), the largest-first group order falling back to plain
  order when there are more local groups than threads, and the two-workgroup
  trans_ragged_dot variant for more than 512 local groups.
* 1024 groups with a 600-group window at offset 424 and a valid-row limit.
* Every tile shape on the 1024-group window case.

Sizes are small (k, n of a few hundred) so the oracle finishes in seconds;
group sizes are a seeded multinomial with a quarter of the groups empty.
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bf16_normal, bits
from tests.gpu_util import assert_bf16_is_rne_of_f32, assert_gemm_close, is_pos_zero, is_sentinel, say, sentinel

pytestmark = pytest.mark.gpu

DEV = "cuda"
G = 1024


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def sizes():
    empty = np.random.default_rng(11).permutation(G)[: G // 4]
    return workloads.random_sizes(G, 9000, seed=12, empty=empty)


CASES = [  # (offset, num_local, limit cut from the sum of sizes)
    (None, G, None),
    (424, 600, 333),
]


def check_forward(x, w, gs_host, off, gl, limit, trans_rhs, what):
    m = x.shape[0]
    n = w.shape[1] if trans_rhs else w.shape[2]
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    o32 = sentinel((m, n), torch.float32)
    o16 = sentinel((m, n), torch.bfloat16)
    rd.ragged_dot(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o32)
    rd.ragged_dot(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o16)
    torch.cuda.synchronize()
    lb, lo, hi, L = oracle.boundaries(gs_host, m, off, gl, limit)
    ref = oracle.ragged_dot(bits(x), bits(w), gs_host, off, limit, trans_rhs)
    assert_gemm_close(o32[:L].cpu().numpy(), ref, what)
    assert_bf16_is_rne_of_f32(o16[:L], o32[:L], what)
    assert bool(is_pos_zero(o32[:lo]).all()) and bool(is_pos_zero(o32[hi:L]).all()), what + ": rows outside window"
    assert bool(is_sentinel(o32[L:]).all()) and bool(is_sentinel(o16[L:]).all()), what + ": rows >= L written"


def check_trans(x, dy, gs_host, off, gl, limit, what):
    k, n = x.shape[1], dy.shape[1]
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    d32 = sentinel((gl, k, n), torch.float32)
    d16 = sentinel((gl, k, n), torch.bfloat16)
    rd.trans_ragged_dot(x, dy, gs, gl, offt, limt, out=d32)
    rd.trans_ragged_dot(x, dy, gs, gl, offt, limt, out=d16)
    torch.cuda.synchronize()
    ref = oracle.trans_ragged_dot(bits(x), bits(dy), gs_host, gl, off, limit)
    assert_gemm_close(d32.cpu().numpy(), ref, what)
    assert_bf16_is_rne_of_f32(d16, d32, what)
    lb, lo, hi, L = oracle.boundaries(gs_host, x.shape[0], off, gl, limit)
    empty = np.flatnonzero(np.diff(lb) == 0)
    if empty.size:
        sel = torch.from_numpy(empty).to(DEV)
        assert bool(is_pos_zero(d32[sel]).all()) and bool(is_pos_zero(d16[sel]).all()), what + ": empty group dW"


@pytest.mark.parametrize("off,gl,cut", CASES)
@pytest.mark.parametrize("k,n", [(128, 128), (192, 512)])
def test_max_groups_forward_forms(off, gl, cut, k, n):
    gs_host = sizes()
    m = int(gs_host.sum()) + 40
    limit = None if cut is None else int(gs_host.sum()) - cut
    say(f"edges: G={G} off={off} gl={gl} limit={limit} k={k} n={n} forward forms")
    x = bf16_normal((m, k), 1.0, 13, DEV)
    w = bf16_normal((gl, k, n), 0.1, 14, DEV)
    wt = bf16_normal((gl, n, k), 0.1, 15, DEV)
    check_forward(x, w, gs_host, off, gl, limit, False, f"G={G} gl={gl} k={k} n={n} plain")
    check_forward(x, wt, gs_host, off, gl, limit, True, f"G={G} gl={gl} k={k} n={n} trans_rhs")


@pytest.mark.parametrize("off,gl,cut", CASES)
@pytest.mark.parametrize("k,n", [(128, 256), (64, 128)])
def test_max_groups_trans_ragged_dot(off, gl, cut, k, n):
    gs_host = sizes()
    m = int(gs_host.sum()) + 40
    limit = None if cut is None else int(gs_host.sum()) - cut
    say(f"edges: G={G} off={off} gl={gl} limit={limit} k={k} n={n} trans_ragged_dot")
    x = bf16_normal((m, k), 1.0, 16, DEV, nan_rows_from=limit)
    dy = bf16_normal((m, n), 1.0, 17, DEV, nan_rows_from=limit)
    check_trans(x, dy, gs_host, off, gl, limit, f"G={G} gl={gl} k={k} n={n} dW")


@pytest.mark.parametrize("tile", list(range(19)))
def test_max_groups_window_every_tile(tile):
    gs_host = sizes()
    off, gl, cut = CASES[1]
    m = int(gs_host.sum()) + 40
    limit = int(gs_host.sum()) - cut
    say(f"edges: G={G} window every tile: tile {tile}")
    k, n = 128, 256
    x = bf16_normal((m, k), 1.0, 18, DEV, nan_rows_from=limit)
    w = bf16_normal((gl, k, n), 0.1, 19, DEV)
    wt = bf16_normal((gl, n, k), 0.1, 20, DEV)
    dy = bf16_normal((m, n), 1.0, 21, DEV, nan_rows_from=limit)
    with rd.tuning(fwd_tile=tile, trans_tile=tile, decode=False):
        check_forward(x, w, gs_host, off, gl, limit, False, f"tile {tile} plain")
        check_forward(x, wt, gs_host, off, gl, limit, True, f"tile {tile} trans_rhs")
        check_trans(x, dy, gs_host, off, gl, limit, f"tile {tile} dW")

"""GPU tests of the up-projection with the GLU as its epilogue (rd_forward_glu).

The fused kernel must give, bit for bit, what the separate kernels give:
act == rd_glu_fwd(rd_forward(x, wi)) and fused == rd_forward(x, wi) (bf16),
on sentinel-filled outputs (rows >= limit untouched, rows below it outside the
window +0), over windows, limits, empty and ragged groups and every tile shape
the fused path has.  Against the oracle, act is within 1 bf16 ulp of the
oracle's GLU of the GPU's [gate | up] buffer; that buffer is the bf16
ragged_dot output, whose float32 form the ragged_dot tests compare with the
oracle.
"""

import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bits, bf16_normal
from tests.gpu_util import assert_glu_close, is_pos_zero, is_sentinel, say, sentinel

pytestmark = pytest.mark.gpu

DEV = "cuda"
TILES = [None, "0", "2", "8", "14"]  # None: the host's own choice


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def separate_kernels(x, wi, gs, offt, limt, m, h):
    fused = sentinel((m, 2 * h), torch.bfloat16)
    act = sentinel((m, h), torch.bfloat16)
    rd.ragged_dot(x, wi, gs, offt, limt, out=fused)
    rd.glu_fwd(fused, limt, out=act)
    return act, fused


def check_case(x, wi, gs_host, off, limit, what):
    m, h = x.shape[0], wi.shape[2] // 2
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    act = sentinel((m, h), torch.bfloat16)
    fused = sentinel((m, 2 * h), torch.bfloat16)
    rd.ragged_dot_glu(x, wi, gs, offt, limt, act=act, fused=fused)
    act_only = rd.ragged_dot_glu(x, wi, gs, offt, limt, act=sentinel((m, h), torch.bfloat16))
    ref_act, ref_fused = separate_kernels(x, wi, gs, offt, limt, m, h)
    torch.cuda.synchronize()
    _, lo, hi, L = oracle.boundaries(gs_host, m, off, wi.shape[0], limit)
    assert same_bits(fused, ref_fused), what + ": [gate | up] differs from ragged_dot"
    assert same_bits(act, ref_act), what + ": act differs from glu_fwd(ragged_dot)"
    assert same_bits(act_only, act), what + ": act without the [gate | up] output differs"
    assert bool(is_sentinel(act[L:]).all()) and bool(is_sentinel(fused[L:]).all()), what + ": rows >= L written"
    assert bool(is_pos_zero(act[:lo]).all()) and bool(is_pos_zero(act[hi:L]).all()), what + ": rows outside window"
    assert bool(is_pos_zero(fused[:lo]).all()) and bool(is_pos_zero(fused[hi:L]).all()), what
    return act, fused, L


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("window,limit_cut", [(False, None), (True, None), (True, 37), (False, 300)])
def test_fused_equals_separate_kernels(tile, window, limit_cut):
    say(f"ragged_dot_glu tile={tile} window={window} limit_cut={limit_cut}")
    G, k, h = 6, 192, 256
    gs_host = workloads.random_sizes(G, 900, seed=61, empty=(2,))
    m = int(gs_host.sum()) + 40
    off, gl = (1, 3) if window else (None, G)
    x = bf16_normal((m, k), 1.0, 62, DEV)
    wi = bf16_normal((gl, k, 2 * h), 0.08, 63, DEV)
    limit = None if limit_cut is None else int(gs_host.sum()) - limit_cut
    with rd.tuning(fwd_tile=None if tile is None else int(tile)):
        check_case(x, wi, gs_host, off, limit, f"tile {tile}")


@pytest.mark.parametrize("tile", TILES)
def test_fused_against_oracle_glu(tile):
    """act is within 1 bf16 ulp of the oracle's GLU of the [gate | up] buffer, over the valid rows."""
    say(f"ragged_dot_glu oracle tile={tile}")
    G, k, h = 4, 128, 128
    gs_host = workloads.random_sizes(G, 500, seed=71, empty=(0,))
    m = int(gs_host.sum())
    x = bf16_normal((m, k), 2.0, 72, DEV)
    wi = bf16_normal((G, k, 2 * h), 0.5, 73, DEV)
    limit = m - 11
    with rd.tuning(fwd_tile=None if tile is None else int(tile)):
        act, fused, L = check_case(x, wi, gs_host, None, limit, f"oracle tile {tile}")
    assert_glu_close(bits(act)[:L], oracle.glu_fwd(bits(fused), L), "act")


def test_fused_decode_sized_groups():
    """Groups of a few rows (the 64-row tile), with empty groups and a window.  The reference runs
    ragged_dot on the tile kernels too: its split-contraction decode path (taken with a workspace)
    sums in another order, which the ragged_dot tests hold to the GEMM tolerance instead."""
    say("ragged_dot_glu decode-sized groups")
    G, k, h = 32, 256, 384
    gs_host = workloads.random_sizes(G, 96, seed=81, empty=(0, 5, 6, 31))
    m = int(gs_host.sum())
    x = bf16_normal((m, k), 1.0, 82, DEV)
    wi = bf16_normal((24, k, 2 * h), 0.05, 83, DEV)
    with rd.tuning(decode=False):
        check_case(x, wi, gs_host, 4, None, "decode window")


def test_fused_no_rows_is_a_no_op():
    say("ragged_dot_glu m=0")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    wi = bf16_normal((2, 128, 256), 0.1, 91, DEV)
    gs = torch.zeros(2, dtype=torch.int32, device=DEV)
    act, fused = rd.ragged_dot_glu(x, wi, gs, want_fused=True)
    assert act.shape == (0, 128) and fused.shape == (0, 256)


def test_fused_rejects_unsupported_h():
    say("ragged_dot_glu h=64 rejected")
    x = bf16_normal((8, 128), 1.0, 92, DEV)
    wi = bf16_normal((1, 128, 128), 0.1, 93, DEV)
    gs = torch.tensor([8], dtype=torch.int32, device=DEV)
    with pytest.raises(rd.RDError):
        rd.ragged_dot_glu(x, wi, gs)


def test_fused_full_up_projection():
    """m8192 k4096 h1024 g64 Zipf groups: the fused result is the separate kernels' result bit for bit."""
    say("ragged_dot_glu full up-projection")
    d = workloads.make(2, DEV, parts=("x", "w"))
    act, fused = check_case(d["x"], d["w"], d["gs_host"], None, None, "up-projection")[:2]
    assert act.shape == (8192, 1024) and fused.shape == (8192, 2048)

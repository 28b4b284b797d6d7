"""GPU parity of trans_ragged_dot's row split of long groups against the oracle.

A group whose contraction costs at least the mean work per CU is cut into
row chunks; each chunk's tile goes to the workspace as an fp32 partial
and a second kernel adds the partials in chunk order.  The cases below are
built so that the split happens (the workspace header's split count is read
back to prove it) and compare every element with the float64 oracle, the bf16
result with RNE of the float32 one, and repeated calls bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bits, bf16_normal
from tests.gpu_util import assert_bf16_is_rne_of_f32, assert_gemm_close, is_pos_zero, say, sentinel

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def split_count(ws):
    """Groups the last call split (the first int32 of the workspace header)."""
    return int(ws[:4].view(torch.int32).item())


def run_split(x, dy, gs, gl=None, off=None, limit=None, ws_bytes=None):
    m, k = x.shape
    n = dy.shape[1]
    gl = gs.numel() if gl is None else gl
    size = rd.trans_workspace_size(m, k, n, gl) if ws_bytes is None else ws_bytes
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    d32 = sentinel((gl, k, n), torch.float32)
    d16 = sentinel((gl, k, n), torch.bfloat16)
    rd.trans_ragged_dot(x, dy, gs, gl, offt, limt, out=d32, workspace=ws)
    ns32 = split_count(ws)
    rd.trans_ragged_dot(x, dy, gs, gl, offt, limt, out=d16, workspace=ws)
    torch.cuda.synchronize()
    return d32, d16, ns32, split_count(ws)


CASES = [
    # m, k, n, sizes, window (offset, num_local) or None, limit or None
    (8192, 256, 512, [6000, 310, 0, 502, 377, 250, 400, 353], None, None),          # one long group
    (8192, 256, 512, [3000, 3100, 0, 500, 600, 400, 292, 300], None, None),         # two long groups
    (8192, 1024, 1024, [6100, 300, 200, 600, 0, 400, 392, 200], None, None),        # XCD grid of tiles
    (9000, 256, 264, [100, 5000, 700, 900, 0, 600, 800, 300, 400, 200], (1, 8), 6500),  # window, limit in the group
    (7000, 384, 512, [0, 0, 6511, 1, 0, 3], None, 6800),                            # ragged chunk ends
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_row_split_matches_oracle(case):
    m, k, n, sizes, win, limit = CASES[case]
    say(f"row split case {case}: m={m} k={k} n={n} sizes={sizes} window={win} limit={limit}")
    gs_host = np.array(sizes, dtype=np.int32)
    off, gl = (None, len(sizes)) if win is None else win
    # NaN rows past the valid rows: the chunk bounds must keep them out of dW
    valid = int(min(gs_host.sum(), m if limit is None else limit))
    x = bf16_normal((m, k), 1.0, 100 + case, "cpu", nan_rows_from=valid).to(DEV)
    dy = bf16_normal((m, n), 1.0, 200 + case, "cpu", nan_rows_from=valid).to(DEV)
    gs = torch.tensor(gs_host, dtype=torch.int32, device=DEV)
    d32, d16, ns32, ns16 = run_split(x, dy, gs, gl, off, limit)
    assert ns32 > 0 and ns16 == ns32, f"case {case}: no group was split ({ns32}, {ns16})"
    ref = oracle.trans_ragged_dot(bits(x), bits(dy), gs_host, gl, off, limit)
    assert_gemm_close(d32.cpu().numpy(), ref, f"split case {case}")
    assert_bf16_is_rne_of_f32(d16, d32, f"split case {case}")
    # the same call again: bit for bit
    again = torch.empty_like(d32)
    ws = torch.zeros(rd.trans_workspace_size(m, k, n, gl), dtype=torch.uint8, device=DEV)
    rd.trans_ragged_dot(x, dy, gs, gl, None if off is None else dev_i32(off),
                        None if limit is None else dev_i32(limit), out=again, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int32), d32.view(torch.int32)), f"case {case}: not deterministic"
    # without the split: the same values within float32 summation order
    plain = rd.trans_ragged_dot(x, dy, gs, gl, None if off is None else dev_i32(off),
                                None if limit is None else dev_i32(limit), row_split=False)
    torch.cuda.synchronize()
    assert_gemm_close(plain.cpu().numpy(), d32.cpu().numpy().astype(np.float64), f"case {case} vs unsplit")


def test_small_workspace_splits_fewer_groups():
    """A workspace with room for only a few partial tiles: fewer (or no) splits, same results."""
    say("row split with a small workspace")
    m, k, n = 8192, 256, 512
    gs_host = np.array([3000, 3100, 0, 500, 600, 400, 292, 300], dtype=np.int32)
    x = bf16_normal((m, k), 1.0, 7, "cpu").to(DEV)
    dy = bf16_normal((m, n), 1.0, 8, "cpu").to(DEV)
    gs = torch.tensor(gs_host, dtype=torch.int32, device=DEV)
    ref = oracle.trans_ragged_dot(bits(x), bits(dy), gs_host)
    full = run_split(x, dy, gs)
    tile = 128 * 256 * 4
    assert full[2] == 2
    # the longest group needs 4 chunks x 4 tiles, the next 3 x 4
    for tiles, want in ((0, 0), (4, 0), (16, 1), (27, 1), (28, 2), (1000, 2)):
        d32, d16, ns32, _ = run_split(x, dy, gs, ws_bytes=256 + tiles * tile)
        assert ns32 == want, (tiles, ns32)
        assert_gemm_close(d32.cpu().numpy(), ref, f"workspace of {tiles} tiles")
        assert_bf16_is_rne_of_f32(d16, d32, f"workspace of {tiles} tiles")


def test_full_size_hot_expert_dw_is_split():
    """m32768, k1024, n4096 with one expert holding 60 % of the rows: that expert is split; sampled
    rows against the oracle, bf16 equal to RNE of float32, empty experts +0.  (The Zipf backward's
    largest expert, 9523 rows, stays whole: its tile costs 0.57 of the mean work per CU.)"""
    say("full size: hot-expert dW with the row split")
    gs_host = workloads.hot_expert_sizes()
    m, k, n = 32768, 1024, 4096
    x = bf16_normal((m, k), 1.0, 31, "cpu").to(DEV)
    dy = bf16_normal((m, n), 1.0, 32, "cpu").to(DEV)
    gs = torch.tensor(gs_host, dtype=torch.int32, device=DEV)
    ws = torch.zeros(rd.trans_workspace_size(m, k, n, 64), dtype=torch.uint8, device=DEV)
    dw32 = rd.trans_ragged_dot(x, dy, gs, workspace=ws)
    torch.cuda.synchronize()
    assert split_count(ws) == 1
    dw16 = rd.trans_ragged_dot(x, dy, gs, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    cols = [0, 5, 127, 128, 511, 512, 1023]
    ref = oracle.trans_ragged_dot(bits(x[:, cols].contiguous()), bits(dy), gs_host)
    assert_gemm_close(dw32[:, cols].cpu().numpy(), ref, "hot expert dW (split)")
    assert_bf16_is_rne_of_f32(dw16, dw32, "hot expert dW (split)")
    for j in np.flatnonzero(gs_host == 0):
        assert bool(is_pos_zero(dw32[int(j)]).all()), f"empty group {j} dW not +0"
    d = workloads.make(3, DEV, parts=("x", "dy"))
    ws.zero_()
    rd.trans_ragged_dot(d["x"], d["dy"], d["gs"], out=dw16, workspace=ws)
    torch.cuda.synchronize()
    assert split_count(ws) == 0

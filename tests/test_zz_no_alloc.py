"""The allocation-free forward (rd_forward_noalloc) against rd_forward, through the C ABI.

rd_forward_noalloc computes what rd_forward computes with a workspace; its
decode split path keeps the fp32 partial sums in the library's static
per-GPU scratch instead of a caller workspace.  The same kernels run on the
same split, so outputs must be bit for bit those of rd_forward with a
workspace of rd_forward_workspace_size bytes.  Two calls in a row, the second
with smaller sizes (the scratch keeps the first call's contents), then a
shape that takes the tile kernels (no scratch), each also checked against
the oracle on sampled rows.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bf16_normal, bits
from tests.gpu_util import assert_gemm_close, is_sentinel, say, sentinel

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def noalloc(x, w, gs, off, lim, out):
    lib = rd.library()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    m, k = x.shape
    gl, _, n = w.shape
    st = lib.rd_forward_noalloc(p(x), p(w), p(gs), gs.numel(), p(off), gl, p(lim), p(out),
                                rd.RD_F32 if out.dtype == torch.float32 else rd.RD_BF16, m, k, n,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == rd.RD_OK, lib.rd_status_string(st)


def with_workspace(x, w, gs, off, lim, out):
    m, k = x.shape
    gl, _, n = w.shape
    wsb = rd.library().rd_forward_workspace_size(m, k, n, gl, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    rd.ragged_dot(x, w, gs, off, lim, out=out, workspace=ws)
    return wsb


def compare(x, w, gs_host, off, limit, what, expect_scratch):
    m, k = x.shape
    gl, _, n = w.shape
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    for dtype in (torch.float32, torch.bfloat16):
        a = sentinel((m, n), dtype)
        b = sentinel((m, n), dtype)
        noalloc(x, w, gs, offt, limt, a)
        wsb = with_workspace(x, w, gs, offt, limt, b)
        torch.cuda.synchronize()
        assert (wsb > 0) == expect_scratch, (what, wsb)
        assert wsb <= rd.RD_NOALLOC_SCRATCH_BYTES
        iv = torch.int32 if dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(iv), b.view(iv)), f"{what} {dtype}: differs from rd_forward"
    L = m if limit is None else limit
    assert bool(is_sentinel(a[L:]).all()), what + ": rows >= L written"
    lb, lo, hi, _ = oracle.boundaries(gs_host, m, off, gl, limit)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.integers(lo, max(hi, lo + 1), 64), [lo, max(hi - 1, lo)]]))
    rows = rows[rows < hi]
    if rows.size:
        ref = oracle.ragged_dot(bits(x), bits(w), gs_host, off, limit)
        got = rd.ragged_dot_noalloc(x, w, gs, offt, limt, out=torch.empty((m, n), dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()
        assert_gemm_close(got.cpu().numpy()[rows], ref[rows], what + " vs oracle")


def test_noalloc_matches_rd_forward_twice_then_smaller():
    say("noalloc: decode workload (m512 k4096 n1536 g128)")
    d = workloads.make(5, DEV, parts=("x", "w"))
    compare(d["x"], d["w"], d["gs_host"], None, None, "decode workload", True)
    say("noalloc: second call, smaller (m300 k512 n768 g64, window 8..56, limit)")
    gs_host = workloads.random_sizes(64, 300, seed=5, empty=(0, 9, 10, 63))
    m = int(gs_host.sum()) + 12
    x = bf16_normal((m, 512), 1.0, 6, DEV)
    w = bf16_normal((48, 512, 768), 0.05, 7, DEV)
    compare(x, w, gs_host, 8, int(gs_host.sum()) - 20, "smaller decode-sized call", True)
    say("noalloc: tile-path shape (m2000 k256 n384 g8), no scratch")
    gs_host = workloads.random_sizes(8, 2000, seed=8, empty=(3,))
    x = bf16_normal((2000, 256), 1.0, 9, DEV)
    w = bf16_normal((8, 256, 384), 0.05, 10, DEV)
    compare(x, w, gs_host, None, None, "tile path", False)

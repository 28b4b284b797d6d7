"""GPU parity of the fp8 (E4M3) ragged_dot, plain and trans_rhs forms, against the oracle.

The oracle accumulates the exact products in float64; the kernel in
float32 through the fp8 MFMA, so the GEMM tolerance applies.  Every E4M3
value is exactly a bf16 value, so the bf16 kernel on the widened inputs is
a second, independent reference (same tolerance).
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd, workloads
from tests.gpu_util import (assert_bf16_is_rne_of_f32, assert_gemm_close, is_pos_zero, is_sentinel, say,
                            sentinel)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def fp8_normal(shape, std, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.float8_e4m3fn)


def codes(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


@pytest.mark.parametrize("trans_rhs", [True, False])
@pytest.mark.parametrize("off,limit", [(None, None), (1, None), (None, 300), (2, 250)])
def test_fp8_small(off, limit, trans_rhs):
    say(f"fp8 trans_rhs={trans_rhs} off={off} limit={limit}")
    gs_host = np.array([70, 0, 150, 5, 129, 0, 30], dtype=np.int32)
    m, k, n = int(gs_host.sum()) + 9, 384, 320
    gl = 7 if off is None else 4
    x = fp8_normal((m, k), 1.0, 11)
    w = fp8_normal((gl, n, k) if trans_rhs else (gl, k, n), 0.5, 12)
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    o32 = sentinel((m, n), torch.float32)
    o16 = sentinel((m, n), torch.bfloat16)
    rd.ragged_dot_fp8(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o32)
    rd.ragged_dot_fp8(x, w, gs, offt, limt, trans_rhs=trans_rhs, out=o16)
    # the bf16 kernel on the same (widened) values
    ob = rd.ragged_dot(x.to(torch.bfloat16), w.to(torch.bfloat16), gs, offt, limt, trans_rhs=trans_rhs,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    lb, lo, hi, L = oracle.boundaries(gs_host, m, off, gl, limit)
    ref = oracle.ragged_dot_fp8(codes(x), codes(w), gs_host, off, limit, trans_rhs=trans_rhs)
    assert_gemm_close(o32[:L].cpu().numpy(), ref, "fp8")
    assert_gemm_close(ob[:L].cpu().numpy(), ref, "bf16 of fp8 values")
    outside = torch.ones(L, dtype=torch.bool, device=DEV)
    outside[lo:hi] = False
    assert bool(is_pos_zero(o32[:L][outside]).all())
    assert bool(is_sentinel(o32[L:]).all()) and bool(is_sentinel(o16[L:]).all())
    assert_bf16_is_rne_of_f32(o16[:L], o32[:L], "fp8")


def test_fp8_moe_backward_shape_sampled():
    """dx of the backward workload (m32768, w[64, 1024, 4096]) with fp8 operands, sampled rows."""
    say("fp8 trans_rhs backward shape")
    d = workloads.make(3, DEV, parts=())
    gs_host = d["gs_host"]
    m, n, k = 32768, 1024, 4096
    x = fp8_normal((m, k), 1.0, 21)
    w = fp8_normal((64, n, k), 0.05, 22)
    o32 = rd.ragged_dot_fp8(x, w, d["gs"], trans_rhs=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.integers(0, m, size=96), [0, m - 1]]))
    lb = np.concatenate([[0], np.cumsum(gs_host)])
    owner = np.searchsorted(lb, rows, side="right") - 1
    counts = np.bincount(owner, minlength=64).astype(np.int32)
    xs = codes(x[torch.from_numpy(rows).to(DEV)])
    ref = oracle.ragged_dot_fp8(xs, codes(w), counts)
    assert_gemm_close(o32[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref, "fp8 backward shape")


def test_fp8_plain_up_projection_sampled():
    """The up-projection (m8192, w[64, 4096, 2048], Zipf groups) in the plain form with fp8 operands,
    sampled rows against the oracle; all rows against the bf16 kernel on the widened values."""
    say("fp8 plain up-projection")
    d = workloads.make(2, DEV, parts=())
    gs_host = d["gs_host"]
    m, k, n = 8192, 4096, 2048
    x = fp8_normal((m, k), 1.0, 31)
    w = fp8_normal((64, k, n), 0.05, 32)
    o32 = rd.ragged_dot_fp8(x, w, d["gs"], out_dtype=torch.float32)
    ob = rd.ragged_dot(x.to(torch.bfloat16), w.to(torch.bfloat16), d["gs"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = (o32 - ob).norm() / ob.norm()
    assert float(err) <= 1e-5, f"fp8 vs bf16 kernel on the same values: {float(err):.2e}"
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.integers(0, m, size=64), [0, m - 1]]))
    lb = np.concatenate([[0], np.cumsum(gs_host)])
    owner = np.searchsorted(lb, rows, side="right") - 1
    counts = np.bincount(owner, minlength=64).astype(np.int32)
    xs = codes(x[torch.from_numpy(rows).to(DEV)])
    ref = oracle.ragged_dot_fp8(xs, codes(w), counts, trans_rhs=False)
    assert_gemm_close(o32[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref, "fp8 plain up-projection")


@pytest.mark.parametrize("off,limit", [(None, None), (1, None), (2, 250)])
def test_fp8_trans_ragged_dot_small(off, limit):
    """dw[j] = x_j^T dy_j on fp8 operands against the oracle (float32 output, GEMM tolerance), NaN rows past
    the limit never reaching dw, an empty group +0, bf16 output = RNE of the float32 one."""
    say(f"fp8 trans_ragged_dot off={off} limit={limit}")
    gs_host = np.array([70, 0, 150, 5, 129, 0, 30], dtype=np.int32)
    m, k, n = int(gs_host.sum()) + 9, 192, 320
    gl = 7 if off is None else 4
    x = fp8_normal((m, k), 1.0, 41)
    y = fp8_normal((m, n), 1.0, 42)
    if limit is not None:  # NaN codes past the limit must be removed by selection
        x.view(torch.uint8)[limit:] = 0x7F
        y.view(torch.uint8)[limit:] = 0x7F
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    d32 = sentinel((gl, k, n), torch.float32)
    d16 = sentinel((gl, k, n), torch.bfloat16)
    rd.trans_ragged_dot_fp8(x, y, gs, gl, offt, limt, out=d32)
    rd.trans_ragged_dot_fp8(x, y, gs, gl, offt, limt, out=d16)
    torch.cuda.synchronize()
    ref = oracle.trans_ragged_dot_fp8(codes(x), codes(y), gs_host, gl, off, limit)
    assert_gemm_close(d32.cpu().numpy(), ref, "fp8 trans")
    assert_bf16_is_rne_of_f32(d16, d32, "fp8 trans")
    lb, _, _, _ = oracle.boundaries(gs_host, m, off, gl, limit)
    for j in range(gl):
        if lb[j + 1] == lb[j]:
            assert bool(is_pos_zero(d32[j]).all()) and bool(is_pos_zero(d16[j]).all()), j


def test_fp8_trans_backward_shape_sampled():
    """dW of the backward workload (x [32768, 1024], dy [32768, 4096], 64 groups, 4 empty) with fp8 operands:
    every group's dW rows sampled against the oracle."""
    say("fp8 trans_ragged_dot backward shape")
    d = workloads.make(3, DEV, parts=())
    gs_host = d["gs_host"]
    m, k, n = 32768, 1024, 4096
    x = fp8_normal((m, k), 1.0, 51)
    y = fp8_normal((m, n), 1.0, 52)
    dw = rd.trans_ragged_dot_fp8(x, y, d["gs"])
    torch.cuda.synchronize()
    lb = np.concatenate([[0], np.cumsum(gs_host)])
    rng = np.random.default_rng(5)
    a_rows = np.sort(rng.choice(k, size=3, replace=False))
    xc, yc = codes(x), codes(y)
    for j in range(64):
        r0, r1 = int(lb[j]), int(lb[j + 1])
        got = dw[j][torch.from_numpy(a_rows).to(DEV)].cpu().numpy()
        if r1 == r0:
            assert np.all(got == 0), j
            continue
        ref = oracle.trans_ragged_dot_fp8(xc[r0:r1][:, a_rows], yc[r0:r1], np.array([r1 - r0], dtype=np.int32))[0]
        assert_gemm_close(got, ref, f"fp8 dW group {j}")


SPLIT_CASES = [
    # m, k, n, sizes, window (offset, num_local) or None, limit or None
    (8192, 256, 512, [6000, 310, 0, 502, 377, 250, 400, 353], None, None),             # one long group
    (9000, 256, 272, [100, 5000, 700, 900, 0, 600, 800, 300, 400, 200], (1, 8), 6500),  # window, limit in it
]


@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
def test_fp8_trans_row_split(case):
    """The row split of long groups on fp8 operands: the group is cut into row chunks (read back from the
    workspace header), fp32 partials added in chunk order; every element against the oracle, NaN codes past
    the valid rows kept out, bf16 = RNE(f32), a repeat bitwise equal, the unsplit result close."""
    m, k, n, sizes, win, limit = SPLIT_CASES[case]
    say(f"fp8 row split case {case}: m={m} k={k} n={n} sizes={sizes} window={win} limit={limit}")
    gs_host = np.array(sizes, dtype=np.int32)
    off, gl = (None, len(sizes)) if win is None else win
    valid = int(min(gs_host.sum(), m if limit is None else limit))
    x = fp8_normal((m, k), 1.0, 60 + case)
    y = fp8_normal((m, n), 1.0, 70 + case)
    x.view(torch.uint8)[valid:] = 0x7F
    y.view(torch.uint8)[valid:] = 0x7F
    gs = torch.from_numpy(gs_host).to(DEV)
    offt = None if off is None else dev_i32(off)
    limt = None if limit is None else dev_i32(limit)
    ws = torch.zeros(rd.trans_workspace_size(m, k, n, gl), dtype=torch.uint8, device=DEV)
    d32 = sentinel((gl, k, n), torch.float32)
    d16 = sentinel((gl, k, n), torch.bfloat16)
    rd.trans_ragged_dot_fp8(x, y, gs, gl, offt, limt, out=d32, workspace=ws)
    torch.cuda.synchronize()
    split_groups = int(ws[:4].view(torch.int32).item())
    rd.trans_ragged_dot_fp8(x, y, gs, gl, offt, limt, out=d16, workspace=ws)
    torch.cuda.synchronize()
    assert split_groups > 0, f"case {case}: no group was split"
    ref = oracle.trans_ragged_dot_fp8(codes(x), codes(y), gs_host, gl, off, limit)
    assert_gemm_close(d32.cpu().numpy(), ref, f"fp8 split case {case}")
    assert_bf16_is_rne_of_f32(d16, d32, f"fp8 split case {case}")
    again = torch.empty_like(d32)
    rd.trans_ragged_dot_fp8(x, y, gs, gl, offt, limt, out=again, workspace=ws)
    plain = rd.trans_ragged_dot_fp8(x, y, gs, gl, offt, limt, row_split=False)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int32), d32.view(torch.int32)), f"case {case}: not deterministic"
    assert_gemm_close(plain.cpu().numpy(), d32.cpu().numpy().astype(np.float64), f"fp8 case {case} vs unsplit")

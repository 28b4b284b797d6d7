"""GPU tests of the autograd wrappers (ragged_dot, trans_ragged_dot, the MoE MLP).

* The wrappers run exactly the kernels their backward rules name: results
  equal the hand-composed kernel calls bit for bit.
* The backward rules against the oracle: every gradient compared with the
  oracle evaluated on the same inputs (GEMM tolerance, float32 outputs).
* The MoE MLP end to end against the oracle, stage by stage: each stage's
  oracle result is computed from the GPU's previous-stage bf16 output, so a
  wiring mistake (a wrong operand, transpose or window) cannot hide in the
  accumulated rounding of the stages before it.
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import autograd as ag
from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bf16_normal, bits
from tests.gpu_util import assert_bf16_is_rne_of_f32, assert_gemm_close, assert_glu_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def _mlp_case(seed, window):
    G, d, h, dout_dim = 8, 256, 128, 192
    gs_host = workloads.random_sizes(G, 700, seed=seed, empty=(2,))
    m = int(gs_host.sum()) + 24
    off, gl = (2, 4) if window else (None, G)
    x = bf16_normal((m, d), 1.0, seed + 1, DEV).requires_grad_(True)
    wi = bf16_normal((gl, d, 2 * h), 0.06, seed + 2, DEV).requires_grad_(True)
    wo = bf16_normal((gl, h, dout_dim), 0.08, seed + 3, DEV).requires_grad_(True)
    gs = torch.from_numpy(gs_host).to(DEV)
    return gs_host, gs, x, wi, wo, off, gl, m


@pytest.mark.parametrize("window", [False, True])
@pytest.mark.parametrize("limit_cut", [None, 40])
def test_moe_mlp_equals_composed_kernels_bitwise(window, limit_cut):
    say(f"moe_mlp composed window={window} limit_cut={limit_cut}")
    gs_host, gs, x, wi, wo, off, gl, m = _mlp_case(500, window)
    offt = None if off is None else dev_i32(off)
    L = m if limit_cut is None else int(gs_host.sum()) - limit_cut
    limt = None if limit_cut is None else dev_i32(L)
    out = ag.moe_mlp(x, wi, wo, gs, offt, limt, zero_tail=True)
    dout = bf16_normal(out.shape, 1.0, 509, DEV)
    dx, dwi, dwo = torch.autograd.grad(out, (x, wi, wo), dout)
    torch.cuda.synchronize()
    with torch.no_grad():
        fused = rd.ragged_dot(x, wi, gs, offt, limt)
        act = rd.glu_fwd(fused, limt)
        ref_out = rd.ragged_dot(act, wo, gs, offt, limt)
        d_act = rd.ragged_dot(dout, wo, gs, offt, limt, trans_rhs=True)
        ref_dwo = rd.trans_ragged_dot(act, dout, gs, gl, offt, limt, out_dtype=torch.bfloat16)
        d_fused = rd.glu_bwd(fused, d_act, limt)
        ref_dx = rd.ragged_dot(d_fused, wi, gs, offt, limt, trans_rhs=True)
        ref_dwi = rd.trans_ragged_dot(x, d_fused, gs, gl, offt, limt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert same(out[:L], ref_out[:L]) and same(dx[:L], ref_dx[:L])
    assert same(dwi, ref_dwi) and same(dwo, ref_dwo)
    assert bool((out[L:] == 0).all()) and bool((dx[L:] == 0).all()), "zero_tail rows"


@pytest.mark.parametrize("window", [False, True])
def test_moe_mlp_against_oracle_stage_by_stage(window):
    """Each GEMM stage: the same kernel with a float32 output is within the GEMM tolerance of the oracle
    (fed the GPU's bf16 inputs of that stage), and the layer's bf16 value is the RNE of it; each GLU
    stage is within 1 bf16 ulp of the oracle."""
    say(f"moe_mlp oracle window={window}")
    gs_host, gs, x, wi, wo, off, gl, m = _mlp_case(520, window)
    offt = None if off is None else dev_i32(off)
    lim = int(gs_host.sum()) - 17
    limt = dev_i32(lim)
    out = ag.moe_mlp(x, wi, wo, gs, offt, limt)
    dout = bf16_normal(out.shape, 1.0, 529, DEV)
    dx, dwi, dwo = torch.autograd.grad(out, (x, wi, wo), dout)
    f32 = torch.float32
    with torch.no_grad():  # the layer's intermediate bf16 tensors, and every GEMM again in float32
        fused = rd.ragged_dot(x, wi, gs, offt, limt)
        fused32 = rd.ragged_dot(x, wi, gs, offt, limt, out_dtype=f32)
        act = rd.glu_fwd(fused, limt)
        out32 = rd.ragged_dot(act, wo, gs, offt, limt, out_dtype=f32)
        d_act = rd.ragged_dot(dout, wo, gs, offt, limt, trans_rhs=True)
        d_act32 = rd.ragged_dot(dout, wo, gs, offt, limt, trans_rhs=True, out_dtype=f32)
        dwo32 = rd.trans_ragged_dot(act, dout, gs, gl, offt, limt, out_dtype=f32)
        d_fused = rd.glu_bwd(fused, d_act, limt)
        dx32 = rd.ragged_dot(d_fused, wi, gs, offt, limt, trans_rhs=True, out_dtype=f32)
        dwi32 = rd.trans_ragged_dot(x, d_fused, gs, gl, offt, limt, out_dtype=f32)
    torch.cuda.synchronize()
    L = lim
    xb, wib, wob, doutb = bits(x), bits(wi), bits(wo), bits(dout)
    stages = [
        ("fused", fused[:L], fused32[:L], oracle.ragged_dot(xb, wib, gs_host, off, lim)),
        ("out", out[:L], out32[:L], oracle.ragged_dot(bits(act), wob, gs_host, off, lim)),
        ("d_act", d_act[:L], d_act32[:L], oracle.ragged_dot(doutb, wob, gs_host, off, lim, trans_rhs=True)),
        ("dwo", dwo, dwo32, oracle.trans_ragged_dot(bits(act), doutb, gs_host, gl, off, lim)),
        ("dx", dx[:L], dx32[:L], oracle.ragged_dot(bits(d_fused), wib, gs_host, off, lim, trans_rhs=True)),
        ("dwi", dwi, dwi32, oracle.trans_ragged_dot(xb, bits(d_fused), gs_host, gl, off, lim)),
    ]
    for what, v16, v32, ref in stages:
        assert_gemm_close(v32.cpu().numpy(), ref, what)
        assert_bf16_is_rne_of_f32(v16, v32, what)
    assert_glu_close(bits(act)[:L], oracle.glu_fwd(bits(fused), lim), "act")
    assert_glu_close(bits(d_fused)[:L], oracle.glu_bwd(bits(fused), bits(d_act), lim), "d_fused")


@pytest.mark.parametrize("trans_rhs", [False, True])
def test_ragged_dot_backward_rules(trans_rhs):
    say(f"RaggedDot backward trans_rhs={trans_rhs}")
    G, k, n = 5, 192, 160
    gs_host = workloads.random_sizes(G, 600, seed=31, empty=(1,))
    m = int(gs_host.sum())
    gs = torch.from_numpy(gs_host).to(DEV)
    x = bf16_normal((m, k), 1.0, 32, DEV).requires_grad_(True)
    w = bf16_normal((G, n, k) if trans_rhs else (G, k, n), 0.1, 33, DEV).requires_grad_(True)
    out = ag.ragged_dot(x, w, gs, trans_rhs=trans_rhs)
    dout = bf16_normal(out.shape, 1.0, 34, DEV)
    dx, dw = torch.autograd.grad(out, (x, w), dout)
    with torch.no_grad():
        dx32 = rd.ragged_dot(dout, w, gs, trans_rhs=not trans_rhs, out_dtype=torch.float32)
        dw32 = (rd.trans_ragged_dot(dout, x, gs) if trans_rhs else rd.trans_ragged_dot(x, dout, gs))
    torch.cuda.synchronize()
    xb, wb, db = bits(x), bits(w), bits(dout)
    assert_gemm_close(dx32.cpu().numpy(), oracle.ragged_dot(db, wb, gs_host, trans_rhs=not trans_rhs), "dx")
    ref_dw = oracle.trans_ragged_dot(db, xb, gs_host) if trans_rhs else oracle.trans_ragged_dot(xb, db, gs_host)
    assert_gemm_close(dw32.cpu().numpy(), ref_dw, "dw")
    assert_bf16_is_rne_of_f32(dx, dx32, "dx")
    assert_bf16_is_rne_of_f32(dw, dw32, "dw")


def test_trans_ragged_dot_backward_rules():
    say("TransRaggedDot backward")
    G, k, n = 4, 128, 96
    gs_host = workloads.random_sizes(G, 500, seed=41, empty=(3,))
    m = int(gs_host.sum())
    gs = torch.from_numpy(gs_host).to(DEV)
    x = bf16_normal((m, k), 1.0, 42, DEV).requires_grad_(True)
    y = bf16_normal((m, n), 1.0, 43, DEV).requires_grad_(True)
    z = ag.trans_ragged_dot(x, y, gs)
    dz = bf16_normal(z.shape, 0.1, 44, DEV)
    dx, dy = torch.autograd.grad(z, (x, y), dz)
    with torch.no_grad():
        dx32 = rd.ragged_dot(y, dz, gs, trans_rhs=True, out_dtype=torch.float32)
        dy32 = rd.ragged_dot(x, dz, gs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    xb, yb, dzb = bits(x), bits(y), bits(dz)
    assert_gemm_close(dx32.cpu().numpy(), oracle.ragged_dot(yb, dzb, gs_host, trans_rhs=True), "dx")
    assert_gemm_close(dy32.cpu().numpy(), oracle.ragged_dot(xb, dzb, gs_host), "dy")
    assert_bf16_is_rne_of_f32(dx, dx32, "dx")
    assert_bf16_is_rne_of_f32(dy, dy32, "dy")


@pytest.mark.parametrize("which", ["ragged_dot", "ragged_dot_trans_rhs", "trans_ragged_dot", "moe_mlp"])
def test_input_gradients_are_zero_past_the_limit(which):
    """Rows at or past the limit take no part in the computation: their input gradient is exactly +0,
    whatever the gradient buffer's memory held before (it is recycled from a NaN-filled block)."""
    say(f"gradient tail past the limit: {which}")
    G, k, n = 4, 128, 192
    gs_host = workloads.random_sizes(G, 400, seed=91, empty=(2,))
    m = int(gs_host.sum()) + 30
    L = int(gs_host.sum()) - 57
    gs = torch.from_numpy(gs_host).to(DEV)
    limt = dev_i32(L)
    # leave NaN bit patterns in the allocator's free blocks of the sizes the gradients take
    junk = [torch.full((m, c), float("nan"), dtype=torch.bfloat16, device=DEV) for c in (k, n, 2 * n)]
    del junk
    x = bf16_normal((m, k), 1.0, 92, DEV).requires_grad_(True)
    if which == "moe_mlp":
        wi = bf16_normal((G, k, 2 * n), 0.05, 93, DEV).requires_grad_(True)
        wo = bf16_normal((G, n, k), 0.05, 94, DEV).requires_grad_(True)
        out = ag.moe_mlp(x, wi, wo, gs, None, limt)
        grads = torch.autograd.grad(out, (x,), bf16_normal(out.shape, 1.0, 95, DEV))
    elif which == "trans_ragged_dot":
        y = bf16_normal((m, n), 1.0, 93, DEV).requires_grad_(True)
        z = ag.trans_ragged_dot(x, y, gs, None, None, limt)
        grads = torch.autograd.grad(z, (x, y), bf16_normal(z.shape, 0.1, 95, DEV))
    else:
        trans_rhs = which.endswith("trans_rhs")
        w = bf16_normal((G, n, k) if trans_rhs else (G, k, n), 0.1, 93, DEV).requires_grad_(True)
        out = ag.ragged_dot(x, w, gs, None, limt, trans_rhs=trans_rhs)
        grads = torch.autograd.grad(out, (x,), bf16_normal(out.shape, 1.0, 95, DEV))
    torch.cuda.synchronize()
    for gr in grads:
        assert gr.shape[0] == m
        assert bool((gr[L:].view(torch.int16) == 0).all()), f"{which}: rows past the limit are not +0"
        assert bool(torch.isfinite(gr[:L].float()).all()), f"{which}: non-finite gradient below the limit"


@pytest.mark.parametrize("limit", [None, -5, 0, 17, 300, 1000])
def test_zero_rows_from_limit(limit):
    say(f"zero_rows_from_limit limit={limit}")
    rows = 300
    for dtype, cols in ((torch.bfloat16, 72), (torch.float32, 36), (torch.bfloat16, 4096)):
        buf = bf16_normal((rows, cols), 1.0, 96, DEV).to(dtype)
        before = buf.clone()
        rd.zero_rows_from_limit(buf, None if limit is None else dev_i32(limit))
        torch.cuda.synchronize()
        L = rows if limit is None else min(max(limit, 0), rows)
        assert torch.equal(buf[:L], before[:L])
        assert bool((buf[L:].view(torch.int16 if dtype == torch.bfloat16 else torch.int32) == 0).all())


def test_calls_on_a_side_stream():
    """A call given stream= runs there; outputs and the decode workspace it allocates stay reserved for
    that stream (the caching allocator does not reuse them while the side stream still works)."""
    say("decode ragged_dot on a side stream")
    d = workloads.make(5, DEV, parts=("x", "w"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ref = rd.ragged_dot(d["x"], d["w"], d["gs"])
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        outs.append(rd.ragged_dot(d["x"], d["w"], d["gs"], stream=side))
        # allocations on the current stream in between must not land on the side stream's buffers
        tmp = torch.full((d["m"], d["n"]), 7.0, dtype=torch.bfloat16, device=DEV)
        del tmp
    side.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))

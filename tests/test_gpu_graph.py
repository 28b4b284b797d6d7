"""The whole decode step (ragged_dot -> GLU -> ragged_dot sharing group_sizes) captured in
one HIP graph: capture succeeds only if no call syncs or copies to the host, and
replays stay correct after group_sizes changes on the device between them."""

import numpy as np
import pytest
import torch

from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bf16_normal
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def step(x, wi, wo, gs, h_buf, g_buf, y_buf):
    rd.ragged_dot(x, wi, gs, out=h_buf)
    rd.glu_fwd(h_buf, out=g_buf)
    rd.ragged_dot(g_buf, wo, gs, out=y_buf)


def test_decode_layer_graph_replays_follow_device_group_sizes():
    say("graph capture of decode layer")
    G, m, k, n = 128, 512, 4096, 1536
    d = workloads.make(5, DEV)
    x, wi = d["x"], d["w"]
    wo = bf16_normal((G, n // 2, k), 0.02, 5005, DEV)
    gs = d["gs"].clone()
    h_buf = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    g_buf = torch.empty((m, n // 2), dtype=torch.bfloat16, device=DEV)
    y_buf = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
    step(x, wi, wo, gs, h_buf, g_buf, y_buf)  # eager warm-up (loads the library)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(x, wi, wo, gs, h_buf, g_buf, y_buf)

    alt = [workloads.group_sizes(5, seed=s) for s in (11, 12, 13)]
    alt.append(np.zeros(G, dtype=np.int32))
    alt.append(workloads.group_sizes(5))
    for i, sizes in enumerate(alt):
        new = torch.from_numpy(sizes).to(DEV)
        gs.copy_(new)  # a device-side rewrite, outside the graph
        graph.replay()
        torch.cuda.synchronize()
        got = y_buf.clone()
        # eager reference with fresh buffers
        h2 = torch.empty_like(h_buf)
        g2 = torch.empty_like(g_buf)
        y2 = torch.empty_like(y_buf)
        step(x, wi, wo, gs, h2, g2, y2)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), y2.view(torch.int16)), f"replay {i} differs from eager"
        if sizes.sum() == 0:
            assert bool((got.view(torch.int16) == 0).all())


def test_moe_mlp_training_step_graph_replays_follow_device_group_sizes():
    """Forward and backward of the MoE MLP (autograd wrapper) captured in one graph."""
    from expert_ffn_ragged_amd import autograd as ag

    say("graph capture of the MoE MLP forward + backward")
    G, m, d, h, dout_dim = 16, 1024, 512, 256, 384
    gs = torch.from_numpy(workloads.random_sizes(G, m, seed=70, empty=(3,))).to(DEV)
    x = bf16_normal((m, d), 1.0, 71, DEV).requires_grad_(True)
    wi = bf16_normal((G, d, 2 * h), 0.05, 72, DEV).requires_grad_(True)
    wo = bf16_normal((G, h, dout_dim), 0.06, 73, DEV).requires_grad_(True)
    dout = bf16_normal((m, dout_dim), 1.0, 74, DEV)

    def train_step():
        out = ag.moe_mlp(x, wi, wo, gs)
        return (out,) + torch.autograd.grad(out, (x, wi, wo), dout)

    # warm up and capture on the same side stream, so the leaves' gradient accumulators (created by
    # the warm-up) belong to the stream the captured backward runs on
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            train_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        captured = train_step()

    sizes = [workloads.random_sizes(G, m, seed=s, empty=e) for s, e in ((80, ()), (81, (0, 5)), (82, (15,)))]
    sizes.append(np.array([m] + [0] * (G - 1), dtype=np.int32))
    for i, sz in enumerate(sizes):
        gs.copy_(torch.from_numpy(sz).to(DEV))  # a device-side rewrite, outside the graph
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in captured]
        with torch.cuda.stream(side):  # the eager reference on the stream the accumulators belong to
            want = train_step()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "dx", "dwi", "dwo"), got, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {i}: {name} differs from eager"


def test_window_limit_forward_graph_replays_follow_device_scalars():
    """A window+limit forward (the 128 x 256 eight-wave tile, whose window calls zero the rows outside the
    window between their contraction steps) captured once and replayed after device-side rewrites of
    group_sizes, the window offset and the limit; every replay bitwise equal to eager into a fresh
    buffer filled the same way."""
    say("graph capture of a window+limit forward")
    G, gl, m, k, n = 16, 4, 6144, 256, 512
    x = bf16_normal((m, k), 1.0, 90, DEV)
    w = bf16_normal((gl, k, n), 0.05, 91, DEV)
    gs = torch.from_numpy(workloads.random_sizes(G, m - 200, seed=92, empty=(3,))).to(DEV)
    off = torch.tensor([2], dtype=torch.int32, device=DEV)
    lim = torch.tensor([m - 500], dtype=torch.int32, device=DEV)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    with rd.tuning(fwd_tile=14):
        rd.ragged_dot(x, w, gs, off, lim, out=out)  # eager warm-up
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            rd.ragged_dot(x, w, gs, off, lim, out=out)
    cases = [(workloads.random_sizes(G, m - 200, seed=93), 0, m), (workloads.random_sizes(G, m, seed=94), 5, 3000),
             (workloads.random_sizes(G, m - 1000, seed=95, empty=(6, 7)), 12, 100), (workloads.random_sizes(G, m - 200, seed=92, empty=(3,)), 2, m - 500)]
    for i, (sizes, o, l) in enumerate(cases):
        gs.copy_(torch.from_numpy(sizes).to(DEV))  # device-side rewrites, outside the graph
        off.fill_(o)
        lim.fill_(l)
        out.view(torch.int16).fill_(0x7F7F)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = torch.empty_like(out)
        want.view(torch.int16).fill_(0x7F7F)
        with rd.tuning(fwd_tile=14):
            rd.ragged_dot(x, w, gs, off, lim, out=want)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {i} differs from eager"


@pytest.mark.parametrize("fp8", [False, True])
def test_trans_row_split_graph_replays_follow_device_group_sizes(fp8):
    """trans_ragged_dot with its row-split workspace, captured once.  The split plan is made on the device
    from group_sizes, so replays after device-side rewrites (a hot expert, another hot expert, uniform sizes,
    two long groups) split different groups: the workspace header (split count, first split group) matches an
    eager call's, the hot expert named is the one of the current sizes, and every replay is bitwise equal to
    the eager call with a workspace of its own."""
    say(f"graph capture of trans_ragged_dot with the row split (fp8={fp8})")
    m, k, n, G = 8192, 256, 512, 8
    cases = [np.array(c, dtype=np.int32) for c in ([6000, 310, 0, 502, 377, 250, 400, 353],
                                                   [300, 200, 500, 0, 5500, 700, 492, 500],
                                                   [1024] * 8,
                                                   [3000, 3100, 0, 500, 600, 400, 292, 300])]
    if fp8:
        gen = [torch.Generator(device=DEV).manual_seed(s) for s in (95, 96)]
        x = torch.randn((m, k), generator=gen[0], device=DEV).to(torch.float8_e4m3fn)
        dy = torch.randn((m, n), generator=gen[1], device=DEV).to(torch.float8_e4m3fn)
        call = rd.trans_ragged_dot_fp8
    else:
        x = bf16_normal((m, k), 1.0, 95, DEV)
        dy = bf16_normal((m, n), 1.0, 96, DEV)
        call = rd.trans_ragged_dot
    gs = torch.from_numpy(cases[0]).to(DEV)
    ws = torch.zeros(rd.trans_workspace_size(m, k, n, G), dtype=torch.uint8, device=DEV)
    out = torch.empty((G, k, n), dtype=torch.float32, device=DEV)
    call(x, dy, gs, out=out, workspace=ws)  # eager warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x, dy, gs, out=out, workspace=ws)
    ws_eager = torch.zeros_like(ws)
    for i, sizes in enumerate(cases):
        gs.copy_(torch.from_numpy(sizes).to(DEV))  # device-side rewrite, outside the graph
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, head_replay = out.clone(), ws[:16].view(torch.int32).cpu().tolist()
        want = torch.full_like(out, float("nan"))
        call(x, dy, gs, out=want, workspace=ws_eager)
        torch.cuda.synchronize()
        head_eager = ws_eager[:16].view(torch.int32).cpu().tolist()
        # header: [split groups, BM, BN, then (group, chunks, first chunk) per split group]
        assert head_replay[0] == head_eager[0], f"replay {i}: {head_replay[0]} groups split, eager {head_eager[0]}"
        if head_replay[0] > 0:
            assert head_replay[3] == head_eager[3], f"replay {i}: split group {head_replay[3]}, eager {head_eager[3]}"
        if i in (0, 1):
            assert head_replay[0] > 0 and head_replay[3] == int(np.argmax(sizes)), f"replay {i}: header {head_replay}"
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"replay {i} differs from eager"

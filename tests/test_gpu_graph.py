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

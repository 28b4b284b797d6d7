"""Reentrancy: the library keeps no per-call state, so calls of different entry points
running at the same time on different streams give, bit for bit, what each gives alone
on the default stream."""

import numpy as np
import pytest
import torch

from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bf16_normal
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def test_concurrent_calls_on_four_streams_match_calls_alone():
    say("concurrent forward / trans with row split / fp8 trans_rhs / GLU on four streams")
    G, m, k, n = 8, 6144, 512, 768
    gs = torch.from_numpy(workloads.random_sizes(G, m - 100, seed=120, empty=(5,))).to(DEV)
    hot = torch.tensor([4500, 300, 0, 400, 344, 200, 300, 100], dtype=torch.int32, device=DEV)  # split in dW
    x = bf16_normal((m, k), 1.0, 121, DEV)
    w = bf16_normal((G, k, n), 0.05, 122, DEV)
    dy = bf16_normal((m, n), 1.0, 123, DEV)
    g8 = torch.Generator(device=DEV).manual_seed(124)
    x8 = torch.randn((m, k), generator=g8, device=DEV).to(torch.float8_e4m3fn)
    w8 = (torch.randn((G, n, k), generator=g8, device=DEV) * 0.05).to(torch.float8_e4m3fn)
    fused = bf16_normal((m, 2 * n), 2.0, 125, DEV)
    lim = dev_i32(m - 700)
    off = dev_i32(2)
    ws = torch.zeros(rd.trans_workspace_size(m, k, n, G), dtype=torch.uint8, device=DEV)

    def run(outs, streams, wsp):
        rd.ragged_dot(x, w[:4], gs, off, lim, out=outs[0], stream=streams[0])
        rd.trans_ragged_dot(x, dy, hot, out=outs[1], workspace=wsp, stream=streams[1])
        rd.ragged_dot_fp8(x8, w8, gs, trans_rhs=True, out=outs[2], stream=streams[2])
        rd.glu_fwd(fused, lim, out=outs[3], stream=streams[3])

    def fresh():
        return [torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV),
                torch.full((G, k, n), float("nan"), dtype=torch.float32, device=DEV),
                torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV),
                torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)]

    alone = fresh()
    torch.cuda.synchronize()
    run(alone, [None] * 4, ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) > 0, "the hot group was not split"
    streams = [torch.cuda.Stream() for _ in range(4)]
    for rep in range(3):
        outs = fresh()
        ws2 = torch.zeros_like(ws)
        torch.cuda.synchronize()
        run(outs, streams, ws2)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, alone)):
            assert torch.equal(a.view(torch.int16 if a.dtype != torch.float32 else torch.int32),
                               b.view(torch.int16 if b.dtype != torch.float32 else torch.int32)), f"rep {rep}: op {i} differs"

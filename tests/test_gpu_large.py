"""Operands past 4 GiB: x [1048584, 2048] bf16 is 4.3 GB, beyond what a 32-bit buffer descriptor
spans, so ragged_dot (both forms) and trans_ragged_dot take the register-staged pipeline with 64-bit
addressing.  Checked on samples: forward rows against the oracle run on those rows (a sub-problem with the
same rows in the same groups), dW entries against float64 dots over each group's rows."""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd
from expert_ffn_ragged_amd.workloads import bf16_normal, bits
from tests.gpu_util import assert_gemm_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
M, K, N = (1 << 20) + 8, 2048, 128
SIZES = np.array([300000, 0, 400000, M - 700000 - 1000], dtype=np.int32)  # 1000 rows past the groups


@pytest.fixture(scope="module")
def big():
    assert M * K * 2 >= 1 << 32
    say(f"operands past 4 GiB: x [{M}, {K}] bf16")
    x = torch.randn((M, K), generator=torch.Generator(device=DEV).manual_seed(130), device=DEV).to(torch.bfloat16)
    gs = torch.from_numpy(SIZES).to(DEV)
    yield x, gs
    del x
    torch.cuda.empty_cache()


def sample_rows():
    b = np.concatenate([[0], np.cumsum(SIZES)])
    rows = {0, 1, 299999, 300000, 300001, 700000 - 1, 700000, int(b[-1]) - 1, int(b[-1]), M - 1}
    rows |= set(np.random.default_rng(131).integers(0, M, 40).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("trans_rhs", [False, True])
def test_forward_past_4gib(big, trans_rhs):
    x, gs = big
    say(f"forward past 4 GiB, trans_rhs={trans_rhs}")
    w = bf16_normal((len(SIZES), N, K) if trans_rhs else (len(SIZES), K, N), 0.05, 132, DEV)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    rd.ragged_dot(x, w, gs, trans_rhs=trans_rhs, out_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    rows = sample_rows()
    idx = torch.from_numpy(rows).to(DEV)
    got = out.index_select(0, idx).cpu().numpy()
    xs = bits(x.index_select(0, idx).cpu())
    b = np.concatenate([[0], np.cumsum(SIZES)])
    in_group = rows < b[-1]
    gs_sub = np.array([np.sum((rows >= b[j]) & (rows < b[j + 1])) for j in range(len(SIZES))], dtype=np.int64)
    ref = oracle.ragged_dot(xs[in_group], bits(w.cpu()), gs_sub, trans_rhs=trans_rhs)
    assert_gemm_close(got[in_group], ref, f"forward past 4 GiB, trans_rhs={trans_rhs}")
    assert bool((got[~in_group] == 0).all()), "rows past the groups must be +0"


def test_trans_past_4gib(big):
    x, gs = big
    say("trans_ragged_dot past 4 GiB")
    dy = bf16_normal((M, N), 1.0, 133, DEV)
    dw = torch.full((len(SIZES), K, N), float("nan"), dtype=torch.float32, device=DEV)
    assert rd.trans_workspace_size(M, K, N, len(SIZES)) == 0  # this pipeline never splits
    rd.trans_ragged_dot(x, dy, gs, out=dw)
    torch.cuda.synchronize()
    kidx = np.array([0, 1, 777, 1024, K - 1], dtype=np.int64)
    xs = bits(x.index_select(1, torch.from_numpy(kidx).to(DEV)).cpu())  # [M, 5] columns of x
    ref = oracle.trans_ragged_dot(xs, bits(dy.cpu()), SIZES)              # [G, 5, N]
    got = dw.index_select(1, torch.from_numpy(kidx).to(DEV)).cpu().numpy()
    assert_gemm_close(got, ref, "trans_ragged_dot past 4 GiB")
    assert bool((dw[1] == 0).all()), "the empty group's dW must be +0"

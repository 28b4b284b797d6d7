"""GPU parity of the weighted unsort backward (rd_unsort_bwd_rows) against the oracle.

The gradient is compared bit for bit.  The routing-weight dot adds exact
products in float64 in the kernel's fixed order (each lane its hidden/64
elements in sequence, then a 6-level butterfly over the 64 lanes) and rounds
once to float32, so it is within half a float32 ulp of the exact dot plus
(hidden/64 + 6) float64 unit roundoffs times sum_c |g y|; the test holds it
to that bound and, as the MaxText page's own check of the same kernel does
(PR #5760, the unsort_bwd_rows test), to an absolute 1e-4.  Rows at or past
the limit must keep a sentinel pattern.
"""

import numpy as np
import pytest
import torch

import oracle
from expert_ffn_ragged_amd import rd, workloads
from expert_ffn_ragged_amd.workloads import bf16_normal, bits, f32_uniform
from tests.gpu_util import is_sentinel, say, sentinel

pytestmark = pytest.mark.gpu

DEV = "cuda"
U64 = 2.0 ** -53


def dev_i32(v):
    return torch.tensor([int(v)], dtype=torch.int32, device=DEV)


def run(g, y, w, limit):
    rows, hidden = g.shape
    grad = sentinel((rows, hidden), torch.bfloat16)
    dot = sentinel((rows,), torch.float32)
    rd.unsort_bwd_rows(g, y, w, None if limit is None else dev_i32(limit), grad=grad, dot=dot)
    torch.cuda.synchronize()
    return grad, dot


def check_rows(g, y, w, grad, dot, rows_idx, what):
    """Bitwise gradient and bounded dot error on the given rows (numpy int64 indices)."""
    hidden = g.shape[1]
    idx = torch.from_numpy(rows_idx).to(DEV)
    gb, yb = bits(g[idx]), bits(y[idx])
    wh = w[idx].cpu().numpy()
    ref_grad, ref_dot = oracle.unsort_bwd_rows(gb, yb, wh)
    got_grad = bits(grad[idx])
    nan_ref = (ref_grad & 0x7FFF) > 0x7F80
    assert np.array_equal(got_grad[~nan_ref], ref_grad[~nan_ref]), what + ": gradient bits differ"
    assert np.all((got_grad[nan_ref] & 0x7FFF) > 0x7F80), what + ": NaN gradient expected"
    got_dot = dot[idx].cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_dot)
    assert np.array_equal(np.isnan(got_dot[~fin]), np.isnan(ref_dot[~fin])), what + ": NaN dot mismatch"
    inf = np.isinf(ref_dot)
    assert np.array_equal(got_dot[inf], ref_dot[inf]), what + ": infinite dot mismatch"
    mag = (np.abs(oracle.bf16_bits_to_f64(gb[fin])) * np.abs(oracle.bf16_bits_to_f64(yb[fin]))).sum(axis=1)
    half_ulp = np.spacing(np.abs(ref_dot[fin]).astype(np.float32)).astype(np.float64) / 2
    bound = half_ulp + (hidden / 64 + 6) * U64 * mag + 1e-45
    err = np.abs(got_dot[fin] - ref_dot[fin])
    assert np.all(err <= bound), f"{what}: dot error {err.max() if err.size else 0:.3e} over bound"
    small = np.abs(ref_dot[fin]) < 1e3  # where an absolute tolerance means something for a float32 result
    assert np.all(err[small] <= 1e-4), f"{what}: dot error {err[small].max():.3e} over the page's 1e-4"


@pytest.mark.parametrize("hidden", [256, 4096])
@pytest.mark.parametrize("limit", [0, 1000, 1700, 2048, None])
def test_small_buffer_every_row(hidden, limit):
    rows = 2048
    say(f"unsort rows={rows} hidden={hidden} limit={limit}")
    g = bf16_normal((rows, hidden), 1.0, 300 + hidden, DEV)
    y = bf16_normal((rows, hidden), 1.0, 301 + hidden, DEV)
    w = f32_uniform(rows, -1.0, 1.0, 302 + hidden, DEV)
    grad, dot = run(g, y, w, limit)
    L = rows if limit is None else limit
    if L:
        check_rows(g, y, w, grad, dot, np.arange(L), f"hidden={hidden} limit={limit}")
    assert bool(is_sentinel(grad[L:]).all()) and bool(is_sentinel(dot[L:]).all()), "rows past the limit written"


def test_special_weights_and_values():
    say("unsort special weights")
    rows, hidden = 8, 512
    g = bf16_normal((rows, hidden), 1.0, 310, DEV)
    g.view(torch.int16)[0, :4] = torch.tensor([0x0000, -0x8000, 0x0001, 0x7F80], dtype=torch.int16, device=DEV)
    y = bf16_normal((rows, hidden), 1.0, 311, DEV)
    w = torch.tensor([1.0, -1.0, 2.0 ** 20, 2.0 ** -20, 0.0, 3.4e38, 1e-40, float("nan")], dtype=torch.float32,
                     device=DEV)
    grad, dot = run(g, y, w, None)
    check_rows(g, y, w, grad, dot, np.arange(rows), "special")
    assert torch.equal(grad[0].view(torch.int16), g[0].view(torch.int16))


def test_repeat_runs_are_bitwise_identical():
    say("unsort determinism")
    g = bf16_normal((3000, 1024), 1.0, 320, DEV)
    y = bf16_normal((3000, 1024), 1.0, 321, DEV)
    w = f32_uniform(3000, -1.0, 1.0, 322, DEV)
    a = run(g, y, w, 2500)
    b = run(g, y, w, 2500)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("limit", [0, 1, 1023, 125952, 126156, 225280])
def test_packed_buffer_limits(limit):
    """The packed expert buffer [225280, 4096] with NaN rows past the workload's 126156 valid rows."""
    say(f"unsort packed buffer limit={limit}")
    d = workloads.make(4, DEV, parts=("ug", "uy", "uw"))
    g, y, w = d["ug"], d["uy"], d["uw"]
    grad, dot = run(g, y, w, limit)
    rng = np.random.default_rng(limit + 5)
    L = limit
    if L:
        sample = np.unique(np.concatenate([rng.integers(0, L, size=256), [0, L - 1]]))
        check_rows(g, y, w, grad, dot, sample, f"packed limit={limit}")
        # rows below the workload's valid count hold finite inputs: no NaN may appear there
        fin = min(L, d["limit"])
        assert not bool(torch.isnan(dot[:fin]).any()), "NaN dot on a valid row"
    assert bool(is_sentinel(grad[L:]).all()) and bool(is_sentinel(dot[L:]).all()), "rows past the limit written"

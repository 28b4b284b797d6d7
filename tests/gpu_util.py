"""Shared helpers of the GPU parity tests (comparison rules and sentinels)."""

import sys

import numpy as np
import torch

# GEMM tolerance: relative Frobenius error and elementwise error against the
# float64 oracle, compared on the float32 output (before any bf16 rounding).
REL_FRO = 1e-3
REL_MAX = 4e-3

SENTINEL16 = -1  # 0xFFFF as int16: a bf16 NaN pattern the kernels never produce for valid rows
SENTINEL32 = -1  # 0xFFFFFFFF as int32


def say(msg):
    """Name the case before a GPU step, flushed, so a fault report points at it."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def sentinel(shape, dtype, device="cuda"):
    t = torch.empty(shape, dtype=dtype, device=device)
    if dtype == torch.bfloat16:
        t.view(torch.int16).fill_(SENTINEL16)
    else:
        t.view(torch.int32).fill_(SENTINEL32)
    return t


def is_sentinel(t):
    """Bool tensor (same device): element still holds the sentinel bit pattern."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16) == SENTINEL16
    return t.view(torch.int32) == SENTINEL32


def is_pos_zero(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16) == 0
    return t.view(torch.int32) == 0


def assert_gemm_close(got, ref, what=""):
    """got: float32 array; ref: float64 array (same shape)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape, what)
    assert np.all(np.isfinite(got)), f"non-finite values in {what}"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if scale == 0.0:
        assert np.all(got == 0), f"{what}: reference is zero, output is not"
        return
    err = got - ref
    fro = np.linalg.norm(err) / np.linalg.norm(ref)
    mx = np.max(np.abs(err))
    assert fro <= REL_FRO, f"{what}: relative Frobenius error {fro:.3e} > {REL_FRO}"
    assert mx <= REL_MAX * scale, f"{what}: max |err| {mx:.3e} > {REL_MAX} * {scale:.3e}"


def assert_bf16_is_rne_of_f32(out_bf16, out_f32, what=""):
    """A bf16 output must be the round-to-nearest-even of the same kernel's float32 output."""
    want = out_f32.to(torch.bfloat16).view(torch.int16)
    bad = (out_bf16.view(torch.int16) != want)
    # NaN payloads may differ; both must then be NaN
    both_nan = torch.isnan(out_bf16.float()) & torch.isnan(out_f32)
    n_bad = int((bad & ~both_nan).sum().item())
    assert n_bad == 0, f"{what}: {n_bad} bf16 elements differ from RNE(float32 output)"


def bf16_ulp_distance(a, b):
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(oa - ob)


def bf16_nan(b):
    b = np.asarray(b, dtype=np.int64)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def assert_glu_close(got_bits, want_bits, what=""):
    """GLU rule: within 1 bf16 ulp (+0 == -0), NaN matches NaN, infinities exact."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    want_bits = np.asarray(want_bits, dtype=np.uint16)
    assert got_bits.shape == want_bits.shape, what
    gn, wn = bf16_nan(got_bits), bf16_nan(want_bits)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({int((gn != wn).sum())})"
    fin = ~wn
    ginf = (got_bits & 0x7FFF) == 0x7F80
    winf = (want_bits & 0x7FFF) == 0x7F80
    assert np.array_equal(got_bits[fin & (ginf | winf)], want_bits[fin & (ginf | winf)]), f"{what}: inf mismatch"
    d = bf16_ulp_distance(got_bits[fin], want_bits[fin])
    assert d.size == 0 or d.max() <= 1, f"{what}: {int((d > 1).sum())} elements more than 1 ulp away"

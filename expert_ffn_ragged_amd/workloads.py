"""Seeded synthetic inputs for the five ragged-dot workloads.

This module only draws random numbers: it holds none of the method's
arithmetic, and both the GPU path's tests and the oracle's tests take their
inputs from it.  Recipe:

* group sizes come from ``numpy.random.default_rng(seed)`` (seed = workload
  number unless given): multinomial draws over a uniform or Zipf(s) profile,
  with the stated groups forced empty;
* every float tensor is drawn as float32 normals from its own
  ``torch.Generator`` on the target device (seed ``1000 * workload + id``),
  scaled, and rounded to bf16 by torch's round-to-nearest-even cast;
  generation runs in row chunks of ``_CHUNK`` elements so the float32
  temporaries stay small;
* "NaN rows" (the unused tail of a packed expert buffer) are filled with the
  bf16 quiet-NaN pattern 0x7FC0.

No public benchmark or dataset is involved; the shapes, distributions and
sparsity follow the workloads the pages describe (a packed buffer of 225280
rows with 126156 valid rows, 256 experts with a local window of 32, MoE
up/down projections, a decode step of 64 tokens with top-8 routing).
"""

import math

import numpy as np
import torch

_CHUNK = 1 << 26  # elements per float32 generation chunk

# Tensor ids inside a workload, used to derive per-tensor seeds.
_X, _W, _DY, _FUSED, _DOUT, _UG, _UY, _UW = 1, 2, 3, 4, 5, 6, 7, 8

WORKLOADS = {
    1: dict(name="tiny m256 k128 n256 g4", m=256, k=128, n=256, G=4),
    2: dict(name="moe up-proj m8192 k4096 n2048 g64 zipf1.1", m=8192, k=4096, n=2048, G=64),
    3: dict(name="moe backward m32768 w[64,1024,4096] zipf1.1 4 empty", m=32768, k=1024, n=4096, G=64),
    4: dict(name="window+limit G256 off96 gl32 buffer225280x4096 limit126156",
            m=225280, k=4096, n=1024, G=256, offset=96, num_local=32, limit=126156),
    5: dict(name="decode 64tok top8 m512 k4096 n1536 g128 30pct empty", m=512, k=4096, n=1536, G=128),
}


def zipf_probs(G, s, rng):
    """Finite Zipf profile p_r ~ r^-s over ranks 1..G, assigned to groups by a seeded permutation."""
    p = np.arange(1, G + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    probs = np.empty(G, dtype=np.float64)
    probs[rng.permutation(G)] = p
    return probs


def multinomial_sizes(total, probs, rng):
    probs = np.asarray(probs, dtype=np.float64)
    probs = probs / probs.sum()
    return rng.multinomial(total, probs).astype(np.int32)


def group_sizes(workload, seed=None, empty_at=1):
    """int32 group sizes of a workload (host array; upload it to make it device-resident)."""
    rng = np.random.default_rng(workload if seed is None else seed)
    if workload == 1:
        probs = np.full(4, 1.0)
        probs[empty_at] = 0.0
        return multinomial_sizes(256, probs, rng)
    if workload == 2:
        return multinomial_sizes(8192, zipf_probs(64, 1.1, rng), rng)
    if workload == 3:
        probs = zipf_probs(64, 1.1, rng)
        probs[[0, 17, 18, 63]] = 0.0
        return multinomial_sizes(32768, probs, rng)
    if workload == 4:
        return multinomial_sizes(126156, np.full(256, 1.0), rng)
    if workload == 5:
        probs = np.full(128, 1.0)
        probs[rng.permutation(128)[:38]] = 0.0
        return multinomial_sizes(512, probs, rng)
    raise ValueError(f"unknown workload {workload}")


def hot_expert_sizes(total=32768, hot_rows=19660, hot=5, G=64, s=1.1, seed=11):
    """Group sizes with one hot expert: ``hot_rows`` rows in group ``hot``, the rest Zipf(s) over the
    other G - 1 groups (the backward's 32768 rows with 60 % in one expert, by default)."""
    rng = np.random.default_rng(seed)
    rest = multinomial_sizes(total - hot_rows, zipf_probs(G - 1, s, rng), rng)
    return np.concatenate([rest[:hot], [hot_rows], rest[hot:]]).astype(np.int32)


def hot_window_sizes(G=256, total=126156, lo=96, hi=128, s=1.1, seed=44):
    """The packed buffer's valid rows over G groups with Zipf(s) shares whose heaviest hi - lo ranks sit
    in the window [lo, hi) (in a seeded order), the other ranks on the other groups."""
    rng = np.random.default_rng(seed)
    p = np.arange(1, G + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    inside = lo + rng.permutation(hi - lo)
    outside = np.concatenate([np.arange(0, lo), np.arange(hi, G)])[rng.permutation(G - (hi - lo))]
    probs = np.empty(G, dtype=np.float64)
    probs[inside] = p[:hi - lo]
    probs[outside] = p[hi - lo:]
    return multinomial_sizes(total, probs, rng)


def random_sizes(G, total, seed, empty=()):
    """Uniform multinomial sizes with the listed groups forced empty (for sweeps)."""
    rng = np.random.default_rng(seed)
    probs = np.full(G, 1.0)
    probs[list(empty)] = 0.0
    return multinomial_sizes(total, probs, rng)


def bf16_normal(shape, std, seed, device="cpu", nan_rows_from=None):
    """bf16 tensor of N(0, std^2) draws; rows ``>= nan_rows_from`` hold NaN."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    flat = out.view(-1)
    total = flat.numel()
    start = 0
    while start < total:
        cnt = min(_CHUNK, total - start)
        tmp = torch.randn(cnt, generator=gen, device=device, dtype=torch.float32)
        tmp.mul_(std)
        flat[start : start + cnt].copy_(tmp)
        start += cnt
    if nan_rows_from is not None and nan_rows_from < shape[0]:
        out[nan_rows_from:].view(torch.int16).fill_(0x7FC0)
    return out


def f32_uniform(n, lo, hi, seed, device="cpu", nan_from=None):
    """float32 tensor of U[lo, hi) draws from its own generator; entries ``>= nan_from`` hold NaN."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.rand(int(n), generator=gen, device=device, dtype=torch.float32)
    out.mul_(hi - lo).add_(lo)
    if nan_from is not None and nan_from < n:
        out[nan_from:] = float("nan")
    return out


def make(workload, device="cpu", parts=("x", "w", "dy"), seed=None):
    """Inputs of one workload as a dict of tensors (bf16 on ``device``; ``gs`` int32 on ``device``).

    Keys: ``gs`` (and ``gs_host``), plus the requested parts among
    ``x``, ``w``, ``dy``, ``fused``, ``d_out``, and the scalars of the workload.
    Workload 4 also offers the weighted-unsort-backward inputs: ``ug`` (the
    gathered gradient) and ``uy`` (the expert outputs), both ``[m, k]`` bf16
    N(0, 1), and ``uw`` (routing weights, ``[m]`` float32 U[-1, 1)), all NaN
    past the limit.
    """
    cfg = dict(WORKLOADS[workload])
    base = 1000 * (workload if seed is None else seed)
    gs = group_sizes(workload, seed)
    d = dict(cfg)
    d["gs_host"] = gs
    d["gs"] = torch.from_numpy(gs.copy()).to(device)
    m, k, n, G = cfg["m"], cfg["k"], cfg["n"], cfg["G"]
    limit = cfg.get("limit")
    if workload == 1:
        std = 1.0 / math.sqrt(k)
        if "x" in parts:
            d["x"] = bf16_normal((m, k), std, base + _X, device)
        if "w" in parts:
            d["w"] = bf16_normal((G, k, n), std, base + _W, device)
        if "dy" in parts:
            d["dy"] = bf16_normal((m, n), std, base + _DY, device)
        return d
    if workload == 2:
        if "x" in parts:
            d["x"] = bf16_normal((m, k), 1.0, base + _X, device)
        if "w" in parts:
            d["w"] = bf16_normal((G, k, n), 0.02, base + _W, device)
        if "dy" in parts:
            d["dy"] = bf16_normal((m, n), 1.0, base + _DY, device)
        return d
    if workload == 3:
        # dx = ragged_dot(dy, w, trans_rhs) with w[g, n_out=k, n]; dW = trans_ragged_dot(x, dy).
        if "x" in parts:
            d["x"] = bf16_normal((m, k), 1.0, base + _X, device)
        if "w" in parts:
            d["w"] = bf16_normal((G, k, n), 0.02, base + _W, device)
        if "dy" in parts:
            d["dy"] = bf16_normal((m, n), 1.0, base + _DY, device)
        return d
    if workload == 4:
        gl = cfg["num_local"]
        if "x" in parts:
            d["x"] = bf16_normal((m, k), 1.0, base + _X, device, nan_rows_from=limit)
        if "w" in parts:
            d["w"] = bf16_normal((gl, k, n), 0.02, base + _W, device)
        if "fused" in parts:
            d["fused"] = bf16_normal((m, 2 * n), 1.0, base + _FUSED, device, nan_rows_from=limit)
        if "d_out" in parts:
            d["d_out"] = bf16_normal((m, n), 1.0, base + _DOUT, device, nan_rows_from=limit)
        if "ug" in parts:
            d["ug"] = bf16_normal((m, k), 1.0, base + _UG, device, nan_rows_from=limit)
        if "uy" in parts:
            d["uy"] = bf16_normal((m, k), 1.0, base + _UY, device, nan_rows_from=limit)
        if "uw" in parts:
            d["uw"] = f32_uniform(m, -1.0, 1.0, base + _UW, device, nan_from=limit)
        return d
    if workload == 5:
        if "x" in parts:
            d["x"] = bf16_normal((m, k), 1.0, base + _X, device)
        if "w" in parts:
            d["w"] = bf16_normal((G, k, n), 0.02, base + _W, device)
        return d
    raise ValueError(f"unknown workload {workload}")


def bits(t):
    """A bf16 tensor's bit patterns as a host numpy uint16 array."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)

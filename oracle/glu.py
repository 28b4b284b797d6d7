"""Oracle for the limit-aware silu(gate) * up GLU, forward and backward (test infrastructure only).

From MaxText PR #5760 "397B v7x trainer: MoE wo FSDP sharding and
valid-rows-only MoE kernels", the commit on valid rows:

* the fused buffer holds gate and up side by side, ``[rows, 2h]`` as
  ``[gate | up]``; only rows ``[0, limit)`` are processed, the rest are
  neither read nor written;
* the forward is evaluated in float32 with the op sequence negate, exp, + 1,
  divide, multiply, and only the output is rounded to bf16;
* the backward writes ``[d_gate | d_up]`` in one pass, rounded once, and maps
  -0 to +0.

Readings where the page is silent: it prints no backward formula; this
oracle uses the derivative of ``g * sigmoid(g) * u`` in float32,
``d_up = d * silu(g)`` and ``d_gate = d * u * s * (1 + g * (1 - s))`` with
``s = 1 / (1 + exp(-g))``, evaluated left to right; the -0 -> +0 map applies
to both halves of the backward and not to the forward.  ``exp`` is the
float64 exponential rounded to float32 (the correctly rounded float32 value
in all but astronomically rare ties).
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits

_ONE = np.float32(1.0)


def _limit(limit, rows):
    return rows if limit is None else min(max(int(limit), 0), int(rows))


def _exp_neg_f32(g):
    """float32 exp(-g): negate (exact), exponentiate in float64, round to float32."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.exp(-(g.astype(np.float64))).astype(np.float32)


def glu_fwd(fused, limit=None):
    """GLU forward: uint16 ``[rows, 2h]`` -> uint16 ``[L, h]`` bf16 bits.

    ``out = bf16(g / (1 + exp(-g)) * u)`` evaluated in float32 in the page's
    order (negate, exp, + 1, divide, multiply); IEEE signs are kept.
    """
    fused = np.asarray(fused, dtype=np.uint16)
    rows, two_h = fused.shape
    if two_h % 2:
        raise ValueError("fused width must be even")
    h = two_h // 2
    L = _limit(limit, rows)
    g = bf16_bits_to_f32(fused[:L, :h])
    u = bf16_bits_to_f32(fused[:L, h:])
    with np.errstate(over="ignore", invalid="ignore", divide="ignore", under="ignore"):
        e = _exp_neg_f32(g)
        den = e + _ONE
        s = g / den
        o = s * u
    return f32_to_bf16_bits(o)


def glu_bwd(fused, d_out, limit=None):
    """GLU backward: (``[rows, 2h]``, ``[rows, h]``) -> uint16 ``[L, 2h]`` as ``[d_gate | d_up]``.

    In float32: ``s = 1/(1+exp(-g))``, ``d_up = d * (g/(1+exp(-g)))``,
    ``d_gate = ((d*u)*s) * (1 + g*(1 - s))``; each rounded once to bf16, then
    the -0 pattern (0x8000) becomes +0 (0x0000) in both halves.
    """
    fused = np.asarray(fused, dtype=np.uint16)
    d_out = np.asarray(d_out, dtype=np.uint16)
    rows, two_h = fused.shape
    h = two_h // 2
    if d_out.shape != (rows, h):
        raise ValueError("d_out must be [rows, h]")
    L = _limit(limit, rows)
    g = bf16_bits_to_f32(fused[:L, :h])
    u = bf16_bits_to_f32(fused[:L, h:])
    d = bf16_bits_to_f32(d_out[:L])
    with np.errstate(over="ignore", invalid="ignore", divide="ignore", under="ignore"):
        e = _exp_neg_f32(g)
        den = e + _ONE
        sig = _ONE / den
        silu = g / den
        d_up = d * silu
        d_gate = ((d * u) * sig) * (_ONE + g * (_ONE - sig))
    out = np.concatenate([f32_to_bf16_bits(d_gate), f32_to_bf16_bits(d_up)], axis=1)
    out[out == 0x8000] = 0
    return out

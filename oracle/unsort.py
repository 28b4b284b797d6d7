"""Oracle for the limit-aware weighted unsort backward (test infrastructure only).

From MaxText PR #5760 "397B v7x trainer: MoE wo FSDP sharding and
valid-rows-only MoE kernels", the commit on valid rows (the
``unsort_bwd_rows`` kernel for the buffered branch of the ring unsort
backward):

* inputs are the incoming gradient gathered into the sorted (packed expert
  buffer) order, ``g [rows, hidden]`` bf16, the expert outputs in the same
  order, ``y [rows, hidden]`` bf16, and one float32 routing weight per row,
  ``w [rows]``;
* the gradient of the expert outputs is ``bf16(f32(g) * w)``: the product
  is formed in float32 and rounded once to bf16;
* the gradient of the routing weights is the float32 row dot
  ``sum_c f32(g[r, c]) * f32(y[r, c])``; the page allows any summation order
  for it (its kernel changes the order and is checked with an absolute
  tolerance of 1e-4);
* only rows ``[0, limit)`` of the packed buffer hold tokens.

Readings of the page: rows at or past ``L = clamp(limit, 0,
rows)`` are neither read nor written (the page's kernel also writes zeros up
to the end of the 1024-row block holding row ``limit - 1``; that is an
artifact of its block size, not part of what it computes; since the page
states that nothing downstream consumes the rows it leaves unwritten, the
plainest contract is to leave them untouched, as the other kernels here do).  The dot is returned
as the float64 sum of the exact products (every product of two bf16 values
is exact in float64), the value any float32 summation order approximates.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, bf16_bits_to_f64, f32_to_bf16_bits


def _limit(limit, rows):
    return rows if limit is None else min(max(int(limit), 0), int(rows))


def unsort_bwd_rows(g, y, w, limit=None):
    """Weighted unsort backward over the valid rows.

    g, y: uint16 bf16 bits ``[rows, hidden]``; w: float32 ``[rows]``.
    Returns ``(grad, dot)``: uint16 ``[L, hidden]`` with
    ``grad = bf16(f32(g) * w[row])`` (one float32 multiply, then RNE), and
    float64 ``[L]`` with ``dot[r] = sum_c g[r, c] * y[r, c]`` (exact
    products, float64 sum).
    """
    g = np.asarray(g, dtype=np.uint16)
    y = np.asarray(y, dtype=np.uint16)
    w = np.asarray(w, dtype=np.float32)
    rows, hidden = g.shape
    if y.shape != g.shape or w.shape != (rows,):
        raise ValueError("g and y must be [rows, hidden] and w [rows]")
    L = _limit(limit, rows)
    gf = bf16_bits_to_f32(g[:L])
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        prod = gf * w[:L, None]  # float32 x float32 -> float32, round to nearest
    grad = f32_to_bf16_bits(prod)
    dot = (bf16_bits_to_f64(g[:L]) * bf16_bits_to_f64(y[:L])).sum(axis=1)
    return grad, dot

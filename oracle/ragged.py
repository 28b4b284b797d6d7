"""Oracle for ragged_dot, its trans_rhs form and trans_ragged_dot (test infrastructure only).

Definitions, from the pages:

* ragged_dot: rows of ``x[m,k]`` are sorted by group; the rows of group i are
  multiplied by ``w[i]`` (``w[g,k,n]``) to give the same rows of ``out[m,n]``
  (SkyRL-tx PR #867 "Integrate ragged_dot pallas kernel with group_offset
  support", the kernel's call sites and the review of its backward rule).
* trans_rhs: ``w`` is ``[g, n, k]`` and the contraction runs over its last
  dimension; the backward rule on the same page uses it as
  ``dx = ragged_dot(y, dz, trans_rhs=True)``.
* trans_ragged_dot: ``x[m,k]`` and ``y[m,n]`` give ``[g,k,n]`` with
  ``out[i] = x_i^T y_i`` over the rows of group i (same page, the
  ``_gpu_trans_ragged_dot_fwd`` signature: x ``[m,k]``, y ``[m,n]``).
* group_offset window: the exclusive cumulative sum of group_sizes gives the
  local shard's first row ``cum[offset]`` and end ``cum[offset + g_local]``,
  ``g_local = rhs.shape[0]``; rows outside the shard are set to zero (same
  page, the suggested ``fast_ragged_dot`` implementation).
* limit: only rows ``[0, limit)`` of a packed expert buffer hold tokens; rows
  at or past it are neither read nor written (MaxText PR #5760 "397B v7x
  trainer: MoE wo FSDP sharding and valid-rows-only MoE kernels", the commit
  on valid rows).

Readings where the pages are silent:

* group sizes are clamped: a negative size counts as 0, and every boundary is
  clamped to ``[0, L]`` where ``L`` is the limit clamped to ``[0, m]``
  (``m`` when absent);
* a window that does not fit (``offset < 0`` or ``offset + g_local > G``) is
  empty: every row below ``L`` is zero and every local dW is zero;
* the masked rows are exact +0.

Arithmetic: bf16 inputs are widened to float64 exactly and each group's
product is one float64 matrix product (numpy ``@``), with no blocking or
reordering beyond that.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64


def boundaries(group_sizes, m, group_offset=None, num_local=None, limit=None):
    """Row boundaries of the local groups.

    Returns ``(lb, lo, hi, L)``: ``lb`` is int64 ``[num_local + 1]`` with local
    group j owning rows ``[lb[j], lb[j+1])``; ``[lo, hi)`` is the window
    (``lo = lb[0]``, ``hi = lb[-1]``); ``L`` is the clamped limit.

    Follows the cumulative-sum window of the SkyRL-tx page's ``fast_ragged_dot``
    (shard_start = cum[offset], shard_end = cum[offset + g_local]), with the
    limit of the MaxText page as an upper clamp.
    """
    gs = np.asarray(group_sizes, dtype=np.int64).reshape(-1)
    G = gs.size
    L = m if limit is None else min(max(int(limit), 0), int(m))
    off = 0 if group_offset is None else int(group_offset)
    gl = G if num_local is None else int(num_local)
    if off < 0 or off + gl > G:
        lb = np.zeros(gl + 1, dtype=np.int64)
        return lb, 0, 0, L
    cum = np.zeros(G + 1, dtype=np.int64)
    cum[1:] = np.cumsum(np.maximum(gs, 0))
    b = np.minimum(cum, L)
    lb = b[off : off + gl + 1].copy()
    return lb, int(lb[0]), int(lb[-1]), L


def ragged_dot(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False, rows=None):
    """ragged_dot in float64.

    x: uint16 bf16 bits ``[m, k]``.  w: uint16 bf16 bits ``[g_local, k, n]``
    (``[g_local, n, k]`` when ``trans_rhs``).  group_sizes: ``[G]`` ints.
    group_offset: int or None.  limit: int or None.

    Returns float64 ``[L, n]``: rows of local group j are ``x_row @ w[j]``,
    every other row below ``L`` is +0.  Rows ``>= L`` are not part of the
    result (the GPU leaves them untouched).  With ``rows`` (an int sequence of
    row indices below ``L``) only those rows are computed, as ``[len(rows), n]``.
    """
    x = np.asarray(x, dtype=np.uint16)
    w = np.asarray(w, dtype=np.uint16)
    m, k = x.shape
    gl = w.shape[0]
    n = w.shape[1] if trans_rhs else w.shape[2]
    if group_offset is None and gl != np.asarray(group_sizes).size:
        raise ValueError("without group_offset, w must hold one matrix per group")
    lb, lo, hi, L = boundaries(group_sizes, m, group_offset, gl, limit)

    def weight(j):
        wj = bf16_bits_to_f64(w[j])
        return wj.T if trans_rhs else wj

    if rows is None:
        out = np.zeros((L, n), dtype=np.float64)
        for j in range(gl):
            s, e = int(lb[j]), int(lb[j + 1])
            if e > s:
                out[s:e] = bf16_bits_to_f64(x[s:e]) @ weight(j)
        return out

    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= L):
        raise ValueError("requested rows must lie in [0, L)")
    out = np.zeros((rows.size, n), dtype=np.float64)
    inside = (rows >= lo) & (rows < hi)
    owner = np.searchsorted(lb, rows, side="right") - 1
    for j in np.unique(owner[inside]):
        sel = np.nonzero(inside & (owner == j))[0]
        out[sel] = bf16_bits_to_f64(x[rows[sel]]) @ weight(int(j))
    return out


def trans_ragged_dot(x, y, group_sizes, num_local=None, group_offset=None, limit=None, k_index=None):
    """trans_ragged_dot in float64: ``out[j] = x_j^T y_j`` per local group.

    x: uint16 bf16 bits ``[m, k]``; y: uint16 bf16 bits ``[m, n]``.
    Returns float64 ``[num_local, k, n]``; a group with no rows (or a window
    that does not fit) gives an all +0 matrix.  With ``k_index`` (an int
    sequence) only those rows of every ``out[j]`` are computed, as
    ``[num_local, len(k_index), n]``.
    """
    x = np.asarray(x, dtype=np.uint16)
    y = np.asarray(y, dtype=np.uint16)
    m, k = x.shape
    n = y.shape[1]
    if y.shape[0] != m:
        raise ValueError("x and y must have the same number of rows")
    G = np.asarray(group_sizes).size
    gl = G if num_local is None else int(num_local)
    lb, _, _, _ = boundaries(group_sizes, m, group_offset, gl, limit)
    cols = np.arange(k) if k_index is None else np.asarray(k_index, dtype=np.int64).reshape(-1)
    out = np.zeros((gl, cols.size, n), dtype=np.float64)
    for j in range(gl):
        s, e = int(lb[j]), int(lb[j + 1])
        if e > s:
            out[j] = bf16_bits_to_f64(x[s:e][:, cols]).T @ bf16_bits_to_f64(y[s:e])
    return out

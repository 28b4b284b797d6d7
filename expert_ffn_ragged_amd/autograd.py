"""torch autograd wrappers over the librd kernels: ragged_dot, trans_ragged_dot and the MoE MLP.

The backward rules are the ones the SkyRL-tx page (PR #867, "Integrate
ragged_dot pallas kernel with group_offset support") states, with its
review's fix for trans_ragged_dot:

* ``out = ragged_dot(x, w)``: ``dx = ragged_dot(dout, w, trans_rhs)`` and
  ``dw = trans_ragged_dot(x, dout)``;
* ``z = trans_ragged_dot(x, y)``: ``dx = ragged_dot(y, dz, trans_rhs)`` and
  ``dy = ragged_dot(x, dz)``.

The MoE MLP (``moe_mlp``) is the expert FFN of the MaxText page (PR #5760,
"397B v7x trainer: MoE wo FSDP sharding and valid-rows-only MoE kernels"):
``fused = ragged_dot(x, wi)`` as ``[gate | up]``, ``act = silu(gate) * up``
(one kernel with the GLU as the GEMM's epilogue where the shapes allow it),
``out = ragged_dot(act, wo)``; its backward keeps the fused buffer as the GLU
residual (``act`` is recomputed from it, as the page's kernel path does) and
runs every step on the GPU kernels.  All of a layer's kernels read the same
device-resident ``group_sizes``; nothing is copied to the host, so forward
and backward can be captured in a HIP graph.

With a ``limit`` (the packed expert buffer's valid rows), rows at or past it
are neither read nor written by the GEMM and GLU kernels.  Those rows of a
forward output are left as allocated unless ``zero_tail`` is set (the
MaxText page's valid-rows commit: nothing downstream consumes them).  The
gradient of an input there is exactly zero, and that is what comes back: a
device-side kernel (``rd.zero_rows_from_limit``, limit read on the GPU)
writes those rows as +0, so no uninitialised memory reaches accumulation,
clipping or a scatter of the gradient.  Gradients come back in the dtype of
their input (bf16).
"""

import torch

from . import rd


def _none_grads(n):
    return (None,) * n


class RaggedDot(torch.autograd.Function):
    """out[rows of local group j] = x[rows] @ w[j] (trans_rhs: @ w[j].T)."""

    @staticmethod
    def forward(ctx, x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False):
        ctx.save_for_backward(x, w, group_sizes, group_offset, limit)
        ctx.trans_rhs = trans_rhs
        return rd.ragged_dot(x, w, group_sizes, group_offset, limit, trans_rhs=trans_rhs)

    @staticmethod
    def backward(ctx, dout):
        x, w, gs, off, lim = ctx.saved_tensors
        dout = dout.contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0]:
            # d/dx of x @ w is dout @ w^T; with trans_rhs (x @ w^T) it is dout @ w
            dx = rd.zero_rows_from_limit(rd.ragged_dot(dout, w, gs, off, lim, trans_rhs=not ctx.trans_rhs), lim)
        if ctx.needs_input_grad[1]:
            gl = w.shape[0]
            if ctx.trans_rhs:   # w[j] is [n, k]: dw[j] = dout_j^T x_j
                dw = rd.trans_ragged_dot(dout, x, gs, gl, off, lim, out_dtype=w.dtype)
            else:               # w[j] is [k, n]: dw[j] = x_j^T dout_j
                dw = rd.trans_ragged_dot(x, dout, gs, gl, off, lim, out_dtype=w.dtype)
        return (dx, dw) + _none_grads(4)


class TransRaggedDot(torch.autograd.Function):
    """z[j] = x_j^T @ y_j over the rows of local group j; [num_local, k, n]."""

    @staticmethod
    def forward(ctx, x, y, group_sizes, num_local=None, group_offset=None, limit=None, out_dtype=None):
        ctx.save_for_backward(x, y, group_sizes, group_offset, limit)
        return rd.trans_ragged_dot(x, y, group_sizes, num_local, group_offset, limit,
                                   out_dtype=x.dtype if out_dtype is None else out_dtype)

    @staticmethod
    def backward(ctx, dz):
        x, y, gs, off, lim = ctx.saved_tensors
        dz = dz.to(x.dtype).contiguous()
        dx = dy = None
        if ctx.needs_input_grad[0]:
            dx = rd.zero_rows_from_limit(rd.ragged_dot(y, dz, gs, off, lim, trans_rhs=True), lim)  # y_r @ dz[j]^T
        if ctx.needs_input_grad[1]:
            dy = rd.zero_rows_from_limit(rd.ragged_dot(x, dz, gs, off, lim), lim)  # x_r @ dz[j] (the review's fix)
        return (dx, dy) + _none_grads(5)


class MoeMLP(torch.autograd.Function):
    """out = ragged_dot(silu(gate) * up, wo) with [gate | up] = ragged_dot(x, wi)."""

    @staticmethod
    def forward(ctx, x, wi, wo, group_sizes, group_offset=None, limit=None, zero_tail=False):
        m = x.shape[0]
        # one kernel (GEMM + GLU epilogue), except for decode-sized groups, whose split-contraction
        # ragged_dot path streams the weights faster than the fused tile kernel
        if m > 24 * wi.shape[0] and rd.glu_epilogue_supported(m, x.shape[1], wi.shape[2] // 2):
            act, fused = rd.ragged_dot_glu(x, wi, group_sizes, group_offset, limit, want_fused=True)
        else:
            fused = rd.ragged_dot(x, wi, group_sizes, group_offset, limit)
            act = rd.glu_fwd(fused, limit)
        out = torch.zeros((m, wo.shape[2]), dtype=x.dtype, device=x.device) if zero_tail else None
        out = rd.ragged_dot(act, wo, group_sizes, group_offset, limit, out=out)
        ctx.save_for_backward(x, wi, wo, group_sizes, group_offset, limit, fused)
        ctx.zero_tail = zero_tail
        return out

    @staticmethod
    def backward(ctx, dout):
        x, wi, wo, gs, off, lim, fused = ctx.saved_tensors
        dout = dout.contiguous()
        gl = wi.shape[0]
        act = rd.glu_fwd(fused, lim)                                         # recomputed from the residual
        d_act = rd.ragged_dot(dout, wo, gs, off, lim, trans_rhs=True)        # [m, h]
        dwo = rd.trans_ragged_dot(act, dout, gs, gl, off, lim, out_dtype=wo.dtype)
        d_fused = rd.glu_bwd(fused, d_act, lim)                              # [d_gate | d_up]
        dx = None
        if ctx.needs_input_grad[0]:
            dx = rd.zero_rows_from_limit(rd.ragged_dot(d_fused, wi, gs, off, lim, trans_rhs=True), lim)
        dwi = rd.trans_ragged_dot(x, d_fused, gs, gl, off, lim, out_dtype=wi.dtype)
        return (dx, dwi, dwo) + _none_grads(4)


def ragged_dot(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False):
    """Differentiable ragged_dot (gradients for x and w)."""
    return RaggedDot.apply(x, w, group_sizes, group_offset, limit, trans_rhs)


def trans_ragged_dot(x, y, group_sizes, num_local=None, group_offset=None, limit=None, out_dtype=None):
    """Differentiable trans_ragged_dot (gradients for x and y)."""
    return TransRaggedDot.apply(x, y, group_sizes, num_local, group_offset, limit, out_dtype)


def moe_mlp(x, wi, wo, group_sizes, group_offset=None, limit=None, zero_tail=False):
    """Differentiable MoE expert MLP over tokens sorted by expert.

    x: [m, d] bf16; wi: [num_local, d, 2h] bf16 producing [gate | up]; wo: [num_local, h, d_out] bf16;
    group_sizes: [G] int32 on the GPU; group_offset, limit: optional (1,) int32 GPU tensors.
    """
    return MoeMLP.apply(x, wi, wo, group_sizes, group_offset, limit, zero_tail)

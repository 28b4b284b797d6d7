"""Thin ctypes binding over librd.so (include/rd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or a call fails,
an exception is raised.

Device scalars (``group_offset``, ``limit``) are passed as int32 tensors of
shape ``(1,)`` on the GPU, and ``group_sizes`` as an int32 GPU tensor, so a
call never reads device data on the host and can be captured in a HIP graph.
"""

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librd.so")

ABI_VERSION = 8
RD_OK, RD_EINVAL, RD_EUNSUPPORTED, RD_EHIP, RD_ESCRATCH = 0, 1, 2, 3, 4
RD_NOALLOC_SCRATCH_BYTES = 80 << 20
RD_BF16, RD_F32 = 0, 1
_DTYPES = {torch.bfloat16: RD_BF16, torch.float32: RD_F32}

EXPORTS = (
    "rd_abi_version",
    "rd_status_string",
    "rd_forward_workspace_size",
    "rd_forward",
    "rd_forward_noalloc",
    "rd_forward_trans_rhs",
    "rd_forward_trans_rhs_fp8",
    "rd_forward_fp8",
    "rd_forward_glu",
    "rd_trans_workspace_size",
    "rd_trans",
    "rd_trans_fp8",
    "rd_glu_fwd",
    "rd_glu_bwd",
    "rd_unsort_bwd_rows",
    "rd_zero_rows_from_limit",
    "rd_tune_set",
    "rd_tune_tile_count",
)
RD_TUNE_FWD_TILE, RD_TUNE_TRANS_TILE, RD_TUNE_DECODE = 0, 1, 2


class RDError(RuntimeError):
    """A nonzero status from librd.so."""


_lib = None


def library():
    """The loaded librd.so (loaded once, after torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RDError(f"{LIB_PATH} is not built; run `python -m expert_ffn_ragged_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.rd_abi_version.restype = ctypes.c_int
    lib.rd_abi_version.argtypes = []
    lib.rd_status_string.restype = ctypes.c_char_p
    lib.rd_status_string.argtypes = [ctypes.c_int]
    lib.rd_forward_workspace_size.restype = sz
    lib.rd_forward_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    fwd = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i64, i64, i64, vp, sz, vp]
    for name in ("rd_forward", "rd_forward_trans_rhs"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = fwd
    lib.rd_forward_noalloc.restype = ctypes.c_int
    lib.rd_forward_noalloc.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i64, i64, i64, vp]
    lib.rd_forward_trans_rhs_fp8.restype = ctypes.c_int
    lib.rd_forward_trans_rhs_fp8.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i64, i64, i64, vp]
    lib.rd_forward_fp8.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i64, i64, i64, vp]
    lib.rd_forward_glu.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, i64, i64, i64, vp]
    lib.rd_trans_workspace_size.restype = sz
    lib.rd_trans_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.rd_trans.restype = ctypes.c_int
    lib.rd_trans.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i64, i64, i64, vp, sz, vp]
    lib.rd_trans_fp8.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, i64, i64, i64, vp, sz, vp]
    lib.rd_glu_fwd.restype = ctypes.c_int
    lib.rd_glu_fwd.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.rd_glu_bwd.restype = ctypes.c_int
    lib.rd_glu_bwd.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.rd_unsort_bwd_rows.restype = ctypes.c_int
    lib.rd_unsort_bwd_rows.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, vp]
    lib.rd_zero_rows_from_limit.restype = ctypes.c_int
    lib.rd_zero_rows_from_limit.argtypes = [vp, vp, i64, i64, vp]
    lib.rd_tune_set.restype = ctypes.c_int
    lib.rd_tune_set.argtypes = [i32, i32]
    lib.rd_tune_tile_count.restype = ctypes.c_int
    lib.rd_tune_tile_count.argtypes = []
    if lib.rd_abi_version() != ABI_VERSION:
        raise RDError("librd.so ABI version mismatch")
    _lib = lib
    return lib


def _check(status):
    if status != RD_OK:
        raise RDError(library().rd_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _launch(fn, tensors, stream, *args):
    """Call C entry point ``fn(*args, stream)`` with the one GPU that every tensor of the call lives on
    made current (the library sizes its grids, and finds its per-GPU scratch, on the current device);
    ``stream`` None means that GPU's current torch stream."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"operands on {dev} and {t.device}: every tensor of a call must be on one GPU")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream on {stream.device}, operands on {dev}")
    with torch.cuda.device(dev):
        _check(fn(*args, ctypes.c_void_p(stream.cuda_stream)))


def _on_stream(stream, *tensors):
    """Tie tensors allocated here (torch's current stream) to the stream the kernels run on, so the
    caching allocator does not hand their memory out again before that stream is done with them."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def tile_count():
    """Number of grouped-GEMM tile shapes ``tuning`` accepts."""
    return library().rd_tune_tile_count()


@contextlib.contextmanager
def tuning(fwd_tile=None, trans_tile=None, decode=None):
    """Force tile shapes (0 .. tile_count() - 1) or turn the decode split path off (decode=False) for
    the calls made inside the block, for tile sweeps; the built-in choices come back on exit.
    Process-wide (rd_tune_set), so not for concurrent use from several threads."""
    lib = library()
    sets = [(RD_TUNE_FWD_TILE, fwd_tile), (RD_TUNE_TRANS_TILE, trans_tile),
            (RD_TUNE_DECODE, None if decode is None else int(bool(decode)))]
    try:
        for key, val in sets:
            if val is not None:
                _check(lib.rd_tune_set(key, int(val)))
        yield
    finally:
        lib.rd_tune_set(RD_TUNE_FWD_TILE, -1)
        lib.rd_tune_set(RD_TUNE_TRANS_TILE, -1)
        lib.rd_tune_set(RD_TUNE_DECODE, 1)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scalar(t, name):
    if t is None:
        return None
    _need(t, name, torch.int32)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold exactly one int32")
    return t


def ragged_dot(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False,
               out_dtype=torch.bfloat16, out=None, workspace=None, stream=None):
    """out[rows of local group j] = x[rows] @ w[j] (or @ w[j].T with trans_rhs).

    x: [m, k] bf16; w: [num_local, k, n] bf16 ([num_local, n, k] with trans_rhs);
    group_sizes: [G] int32 on the GPU; group_offset, limit: optional (1,) int32
    GPU tensors.  Rows below the limit outside the local window are +0; rows
    at or past the limit are left as they were in ``out`` (uninitialised when
    ``out`` is not given).  ``workspace``: optional uint8 GPU scratch; when the
    sizes call for one (decode shapes) and none of sufficient size is given,
    one is allocated.
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    group_offset = _scalar(group_offset, "group_offset")
    limit = _scalar(limit, "limit")
    m, k = x.shape
    gl = w.shape[0]
    if trans_rhs:
        n, kw = w.shape[1], w.shape[2]
    else:
        kw, n = w.shape[1], w.shape[2]
    if kw != k:
        raise ValueError("contraction sizes of x and w differ")
    fresh = out is None
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _need(out, "out", out.dtype, 2)
    if tuple(out.shape) != (m, n) or out.dtype not in _DTYPES:
        raise ValueError("out must be [m, n] bf16 or float32")
    lib = library()
    ws_bytes = lib.rd_forward_workspace_size(m, k, n, gl, 1 if trans_rhs else 0)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
        _on_stream(stream, workspace)
    if fresh:
        _on_stream(stream, out)
    fn = lib.rd_forward_trans_rhs if trans_rhs else lib.rd_forward
    _launch(fn, (x, w, group_sizes, group_offset, limit, out, workspace if ws_bytes else None), stream,
            _ptr(x), _ptr(w), _ptr(group_sizes), group_sizes.numel(), _ptr(group_offset), gl, _ptr(limit), _ptr(out),
            _DTYPES[out.dtype], m, k, n, _ptr(workspace) if ws_bytes else None, ws_bytes)
    return out


def ragged_dot_noalloc(x, w, group_sizes, group_offset=None, limit=None, out=None, stream=None):
    """ragged_dot (plain form) through rd_forward_noalloc: the library allocates nothing (the decode
    path's partial sums live in its static per-GPU scratch); ``out`` ([m, n] bf16 or float32) should be
    given by callers that cannot allocate.  Calls overlapping on one GPU race on that scratch."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 3)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    group_offset = _scalar(group_offset, "group_offset")
    limit = _scalar(limit, "limit")
    m, k = x.shape
    gl, kw, n = w.shape
    if kw != k:
        raise ValueError("contraction sizes of x and w differ")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
        _on_stream(stream, out)
    _need(out, "out", out.dtype, 2)
    if tuple(out.shape) != (m, n) or out.dtype not in _DTYPES:
        raise ValueError("out must be [m, n] bf16 or float32")
    _launch(library().rd_forward_noalloc, (x, w, group_sizes, group_offset, limit, out), stream,
            _ptr(x), _ptr(w), _ptr(group_sizes), group_sizes.numel(), _ptr(group_offset), gl, _ptr(limit), _ptr(out),
            _DTYPES[out.dtype], m, k, n)
    return out


def ragged_dot_fp8(x, w, group_sizes, group_offset=None, limit=None, trans_rhs=False, out_dtype=torch.bfloat16,
                   out=None, stream=None):
    """fp8 (E4M3) ragged_dot: out[rows of local group j] = x[rows] @ w[j] (trans_rhs: @ w[j].T).

    x: [m, k] torch.float8_e4m3fn; w: [num_local, k, n] (trans_rhs: [num_local, n, k]) float8_e4m3fn;
    float32 accumulation, one rounding to out_dtype.
    """
    _need(x, "x", torch.float8_e4m3fn, 2)
    _need(w, "w", torch.float8_e4m3fn, 3)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    group_offset = _scalar(group_offset, "group_offset")
    limit = _scalar(limit, "limit")
    m, k = x.shape
    if trans_rhs:
        gl, n, kw = w.shape
    else:
        gl, kw, n = w.shape
    if kw != k:
        raise ValueError("contraction sizes of x and w differ")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
        _on_stream(stream, out)
    _need(out, "out", out.dtype, 2)
    if tuple(out.shape) != (m, n) or out.dtype not in _DTYPES:
        raise ValueError("out must be [m, n] bf16 or float32")
    fn = library().rd_forward_trans_rhs_fp8 if trans_rhs else library().rd_forward_fp8
    _launch(fn, (x, w, group_sizes, group_offset, limit, out), stream,
            _ptr(x), _ptr(w), _ptr(group_sizes), group_sizes.numel(), _ptr(group_offset), gl, _ptr(limit), _ptr(out),
            _DTYPES[out.dtype], m, k, n)
    return out


def trans_ragged_dot_fp8(x, dy, group_sizes, num_local=None, group_offset=None, limit=None,
                         out_dtype=torch.float32, out=None, workspace=None, row_split=True, stream=None):
    """fp8 (E4M3) trans_ragged_dot: dw[j] = x_j^T @ dy_j, float32 accumulation, one rounding to out_dtype.

    x: [m, k] and dy: [m, n] torch.float8_e4m3fn; returns [num_local, k, n].  ``workspace`` and
    ``row_split`` as for trans_ragged_dot (the same row split of long groups).
    """
    _need(x, "x", torch.float8_e4m3fn, 2)
    _need(dy, "dy", torch.float8_e4m3fn, 2)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    group_offset = _scalar(group_offset, "group_offset")
    limit = _scalar(limit, "limit")
    m, k = x.shape
    if dy.shape[0] != m:
        raise ValueError("x and dy row counts differ")
    n = dy.shape[1]
    gl = group_sizes.numel() if num_local is None else int(num_local)
    if out is None:
        out = torch.empty((gl, k, n), dtype=out_dtype, device=x.device)
        _on_stream(stream, out)
    _need(out, "out", out.dtype, 3)
    if tuple(out.shape) != (gl, k, n) or out.dtype not in _DTYPES:
        raise ValueError("out must be [num_local, k, n] bf16 or float32")
    lib = library()
    ws_bytes = 0
    if row_split and workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws_bytes = workspace.numel()
    elif row_split:
        ws_bytes = lib.rd_trans_workspace_size(m, k, n, gl)
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
            _on_stream(stream, workspace)
    _launch(lib.rd_trans_fp8, (x, dy, group_sizes, group_offset, limit, out, workspace if ws_bytes else None), stream,
            _ptr(x), _ptr(dy), _ptr(group_sizes), group_sizes.numel(), _ptr(group_offset), gl, _ptr(limit),
            _ptr(out), _DTYPES[out.dtype], m, k, n, _ptr(workspace) if ws_bytes else None, ws_bytes)
    return out


def glu_epilogue_supported(m, k, h):
    """Whether ragged_dot_glu takes these sizes: k % 64 == 0, h % 128 == 0, every operand under 4 GiB."""
    return k % 64 == 0 and h % 128 == 0 and h > 0 and m * k * 2 < 1 << 32 and k * 2 * h * 2 < 1 << 32


def ragged_dot_glu(x, wi, group_sizes, group_offset=None, limit=None, act=None, fused=None, want_fused=False,
                   stream=None):
    """The up-projection with the GLU as its epilogue: act = glu_fwd(ragged_dot(x, wi)), bit for bit.

    x: [m, k] bf16; wi: [num_local, k, 2h] bf16 ([gate | up] columns).  Returns act [m, h] bf16, or
    (act, fused) with the [gate | up] buffer fused [m, 2h] when want_fused (or a fused tensor) is given.
    Requires k % 64 == 0 and h % 128 == 0.
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(wi, "wi", torch.bfloat16, 3)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    group_offset = _scalar(group_offset, "group_offset")
    limit = _scalar(limit, "limit")
    m, k = x.shape
    gl, kw, h2 = wi.shape
    if kw != k or h2 % 2:
        raise ValueError("wi must be [num_local, k, 2h] with x's k")
    h = h2 // 2
    if act is None:
        act = torch.empty((m, h), dtype=torch.bfloat16, device=x.device)
        _on_stream(stream, act)
    _need(act, "act", torch.bfloat16, 2)
    if tuple(act.shape) != (m, h):
        raise ValueError("act must be [m, h]")
    if fused is None and want_fused:
        fused = torch.empty((m, h2), dtype=torch.bfloat16, device=x.device)
        _on_stream(stream, fused)
    if fused is not None:
        _need(fused, "fused", torch.bfloat16, 2)
        if tuple(fused.shape) != (m, h2):
            raise ValueError("fused must be [m, 2h]")
    _launch(library().rd_forward_glu, (x, wi, group_sizes, group_offset, limit, act, fused), stream,
            _ptr(x), _ptr(wi), _ptr(group_sizes), group_sizes.numel(), _ptr(group_offset), gl, _ptr(limit),
            _ptr(act), _ptr(fused), m, k, h)
    return act if fused is None else (act, fused)


def trans_ragged_dot(x, dy, group_sizes, num_local=None, group_offset=None, limit=None,
                     out_dtype=torch.float32, out=None, workspace=None, row_split=True, stream=None):
    """dw[j] = x_j^T @ dy_j over the rows of local group j; [num_local, k, n].

    ``workspace``: optional uint8 GPU scratch for the row split of long groups, used as given (a
    smaller one than ``rd_trans_workspace_size`` splits fewer groups); without it one of that size is
    allocated.  ``row_split=False`` passes no workspace (no group is split).
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(dy, "dy", torch.bfloat16, 2)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    group_offset = _scalar(group_offset, "group_offset")
    limit = _scalar(limit, "limit")
    m, k = x.shape
    if dy.shape[0] != m:
        raise ValueError("x and dy must have the same rows")
    n = dy.shape[1]
    gl = group_sizes.numel() if num_local is None else int(num_local)
    fresh = out is None
    if out is None:
        out = torch.empty((gl, k, n), dtype=out_dtype, device=x.device)
    _need(out, "out", out.dtype, 3)
    if tuple(out.shape) != (gl, k, n) or out.dtype not in _DTYPES:
        raise ValueError("out must be [num_local, k, n] bf16 or float32")
    lib = library()
    ws_bytes = 0
    if row_split and workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws_bytes = workspace.numel()
    elif row_split:
        ws_bytes = lib.rd_trans_workspace_size(m, k, n, gl)
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
            _on_stream(stream, workspace)
    if fresh:
        _on_stream(stream, out)
    _launch(lib.rd_trans, (x, dy, group_sizes, group_offset, limit, out, workspace if ws_bytes else None), stream,
            _ptr(x), _ptr(dy), _ptr(group_sizes), group_sizes.numel(), _ptr(group_offset), gl, _ptr(limit),
            _ptr(out), _DTYPES[out.dtype], m, k, n, _ptr(workspace) if ws_bytes else None, ws_bytes)
    return out


def trans_workspace_size(m, k, n, num_local):
    """Bytes of workspace that let trans_ragged_dot split every group that qualifies (0: none can)."""
    return int(library().rd_trans_workspace_size(m, k, n, num_local))


def glu_fwd(fused, limit=None, out=None, stream=None):
    """out[r, c] = bf16(silu(gate) * up) for rows r < limit; fused is [rows, 2h] as [gate | up]."""
    _need(fused, "fused", torch.bfloat16, 2)
    limit = _scalar(limit, "limit")
    rows, two_h = fused.shape
    if two_h % 2:
        raise ValueError("fused width must be even")
    h = two_h // 2
    if out is None:
        out = torch.empty((rows, h), dtype=torch.bfloat16, device=fused.device)
        _on_stream(stream, out)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (rows, h):
        raise ValueError("out must be [rows, h]")
    _launch(library().rd_glu_fwd, (fused, limit, out), stream,
            _ptr(fused), _ptr(limit), _ptr(out), rows, h)
    return out


def glu_bwd(fused, d_out, limit=None, out=None, stream=None):
    """[d_gate | d_up] for rows r < limit, -0 written as +0; returns [rows, 2h] bf16."""
    _need(fused, "fused", torch.bfloat16, 2)
    _need(d_out, "d_out", torch.bfloat16, 2)
    limit = _scalar(limit, "limit")
    rows, two_h = fused.shape
    h = two_h // 2
    if tuple(d_out.shape) != (rows, h):
        raise ValueError("d_out must be [rows, h]")
    if out is None:
        out = torch.empty((rows, two_h), dtype=torch.bfloat16, device=fused.device)
        _on_stream(stream, out)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (rows, two_h):
        raise ValueError("out must be [rows, 2h]")
    _launch(library().rd_glu_bwd, (fused, d_out, limit, out), stream,
            _ptr(fused), _ptr(d_out), _ptr(limit), _ptr(out), rows, h)
    return out


def unsort_bwd_rows(g, y, w, limit=None, grad=None, dot=None, stream=None):
    """(grad, dot) over rows r < limit: grad = bf16(f32(g) * w[r]), dot[r] = sum_c g[r, c] * y[r, c] (float32).

    g, y: [rows, hidden] bf16 in the packed buffer's row order; w: [rows] float32 routing weights.
    Rows at or past the limit are left as they were in ``grad`` and ``dot`` (uninitialised when not given).
    """
    _need(g, "g", torch.bfloat16, 2)
    _need(y, "y", torch.bfloat16, 2)
    _need(w, "w", torch.float32, 1)
    limit = _scalar(limit, "limit")
    rows, hidden = g.shape
    if tuple(y.shape) != (rows, hidden) or w.shape[0] != rows:
        raise ValueError("g and y must be [rows, hidden] and w [rows]")
    if grad is None:
        grad = torch.empty((rows, hidden), dtype=torch.bfloat16, device=g.device)
        _on_stream(stream, grad)
    if dot is None:
        dot = torch.empty((rows,), dtype=torch.float32, device=g.device)
        _on_stream(stream, dot)
    _need(grad, "grad", torch.bfloat16, 2)
    _need(dot, "dot", torch.float32, 1)
    if tuple(grad.shape) != (rows, hidden) or dot.shape[0] != rows:
        raise ValueError("grad must be [rows, hidden] and dot [rows]")
    _launch(library().rd_unsort_bwd_rows, (g, y, w, limit, grad, dot), stream,
            _ptr(g), _ptr(y), _ptr(w), _ptr(limit), _ptr(grad), _ptr(dot), rows, hidden)
    return grad, dot


def zero_rows_from_limit(buf, limit, stream=None):
    """Rows at or past ``limit`` (a (1,) int32 GPU tensor; None: nothing to do) of ``buf`` set to +0,
    in place; ``buf`` is a contiguous GPU tensor whose first dim is the rows.  Returns ``buf``."""
    if limit is None:
        return buf
    limit = _scalar(limit, "limit")
    if buf.device.type != "cuda" or not buf.is_contiguous() or buf.dim() < 1:
        raise ValueError("buf must be a contiguous GPU tensor")
    rows = buf.shape[0]
    row_bytes = buf[0].numel() * buf.element_size() if rows else 16
    _launch(library().rd_zero_rows_from_limit, (buf, limit), stream,
            _ptr(buf) if rows else None, _ptr(limit), rows, row_bytes)
    return buf

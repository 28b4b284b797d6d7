"""Ragged dot (grouped GEMM) for mixture-of-experts expert FFNs on MI355X (gfx950).

The compute lives in ``librd.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rd.h``); :mod:`expert_ffn_ragged_amd.rd` is the thin
ctypes binding over it.  Importing this package loads nothing: the library
is opened on first use of an op, and a missing or unloadable library is an
error, never a fallback.
"""

_OPS = ("ragged_dot", "trans_ragged_dot", "glu_fwd", "glu_bwd", "library", "RDError")


def __getattr__(name):
    if name in _OPS:
        from . import rd

        return getattr(rd, name)
    raise AttributeError(name)

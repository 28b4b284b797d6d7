"""The C-ABI library: it loads, exports every function include/rd.h declares,
shares torch's HIP runtime, and rejects host-visible bad arguments before
launching anything.  Runs without a GPU (no compute call is made)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from expert_ffn_ragged_amd import rd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rd.h")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rd_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rd.LIB_PATH):
        pytest.fail("librd.so is not built (run __graft_entry__.build())")
    return rd.library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(rd.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", rd.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (rd_[a-z_0-9]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_links_the_same_hip_runtime_soname_as_torch():
    needed = subprocess.run(["readelf", "-d", rd.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    assert "libamdhip64.so.7" in needed


def test_version_and_status_strings(lib):
    assert lib.rd_abi_version() == rd.ABI_VERSION == 8
    for s in (0, 1, 2, 3, 99):
        assert isinstance(lib.rd_status_string(s), bytes)


def test_trans_workspace_size(lib):
    """The row-split workspace: a header plus fp32 partial tiles; none when nothing can split."""
    size = lib.rd_trans_workspace_size
    assert size(0, 1024, 4096, 64) == 0                 # no rows
    assert size(1 << 21, 1024, 4096, 64) == 0           # x past 4 GiB: the fallback pipeline never splits
    assert size(100, 12, 64, 4) == 0                    # k not a multiple of 8: rejected sizes
    for m, k, n, gl in ((100, 64, 64, 4), (32768, 1024, 4096, 64), (8192, 4096, 2048, 64)):
        b = size(m, k, n, gl)
        assert b > 256 and (b - 256) % (128 * 128 * 4) == 0, (m, k, n, gl, b)
    # bounded by three partial tiles per workgroup of the grid (at most three workgroups per CU)
    assert size(32768, 1024, 4096, 64) <= 256 + 3 * 3 * 256 * 256 * 256 * 4


def _trans(lib, **kw):
    a = dict(x=16, dy=16, gs=16, G=4, off=None, gl=4, limit=None, dw=16, dt=0, m=8, k=8, n=8, ws=None, ws_bytes=0)
    a.update(kw)
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.rd_trans(v(a["x"]), v(a["dy"]), v(a["gs"]), a["G"], v(a["off"]), a["gl"], v(a["limit"]), v(a["dw"]),
                        a["dt"], a["m"], a["k"], a["n"], v(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None, ws_bytes=4096), rd.RD_EINVAL),   # a workspace size without a workspace
    (dict(ws=24, ws_bytes=4096), rd.RD_EINVAL),     # misaligned workspace
    (dict(dt=7), rd.RD_EINVAL),
    (dict(k=12), rd.RD_EUNSUPPORTED),
])
def test_trans_rejects_before_launch(lib, kw, status):
    assert _trans(lib, **kw) == status


def _fwd(lib, **kw):
    a = dict(x=16, w=16, gs=16, G=4, off=None, gl=4, limit=None, out=16, dt=0, m=8, k=8, n=8)
    a.update(kw)
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.rd_forward(v(a["x"]), v(a["w"]), v(a["gs"]), a["G"], v(a["off"]), a["gl"], v(a["limit"]),
                          v(a["out"]), a["dt"], a["m"], a["k"], a["n"], v(a.get("ws")), a.get("ws_bytes", 0), None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), rd.RD_EINVAL),
    (dict(out=None), rd.RD_EINVAL),
    (dict(gs=None), rd.RD_EINVAL),
    (dict(x=24), rd.RD_EINVAL),            # misaligned
    (dict(gs=18), rd.RD_EINVAL),           # misaligned int32
    (dict(k=12), rd.RD_EUNSUPPORTED),      # k not a multiple of 8
    (dict(n=0), rd.RD_EINVAL),
    (dict(m=-1), rd.RD_EINVAL),
    (dict(dt=7), rd.RD_EINVAL),
    (dict(gl=3), rd.RD_EINVAL),            # no offset needs num_local == num_groups
    (dict(gl=5, off=16), rd.RD_EINVAL),    # num_local > num_groups
    (dict(G=2000, gl=2000), rd.RD_EUNSUPPORTED),
    (dict(G=0, gl=0), rd.RD_EINVAL),
    (dict(m=1 << 31), rd.RD_EUNSUPPORTED),
    (dict(ws=40, ws_bytes=64), rd.RD_EINVAL),  # misaligned workspace
    (dict(m=0), rd.RD_OK),                 # nothing to do, nothing launched
])
def test_forward_rejects_bad_arguments_before_launch(lib, kw, status):
    assert _fwd(lib, **kw) == status


def test_glu_rejects_bad_arguments(lib):
    v = ctypes.c_void_p
    assert lib.rd_glu_fwd(v(16), None, v(16), 4, 12, None) == rd.RD_EUNSUPPORTED
    assert lib.rd_glu_fwd(None, None, v(16), 4, 8, None) == rd.RD_EINVAL
    assert lib.rd_glu_fwd(v(16), None, v(16), 0, 8, None) == rd.RD_OK
    assert lib.rd_glu_bwd(v(16), v(16), None, v(20), 4, 8, None) == rd.RD_EINVAL
    assert lib.rd_glu_bwd(v(16), v(16), v(18), v(16), 4, 8, None) == rd.RD_EINVAL


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(rd, "_lib", None)
    monkeypatch.setattr(rd, "LIB_PATH", "/nonexistent/librd.so")
    with pytest.raises(rd.RDError):
        rd.library()


def test_forward_workspace_size_follows_the_decode_rule(lib):
    """Only decode-sized forward calls (<= 24 rows per local group on average) ask for a workspace."""
    ws = lib.rd_forward_workspace_size(512, 4096, 1536, 128, 0)
    assert 0 < ws <= 256 << 20 and ws % 16 == 0
    assert lib.rd_forward_workspace_size(512, 4096, 1536, 128, 1) == 0      # trans_rhs: none
    assert lib.rd_forward_workspace_size(8192, 4096, 2048, 64, 0) == 0      # prefill-sized groups
    assert lib.rd_forward_workspace_size(512, 4104, 1536, 128, 0) == 0      # k not a multiple of 16
    assert lib.rd_forward_workspace_size(512, 4096, 136, 128, 0) == 0       # n: no 256-column strips
    assert lib.rd_forward_workspace_size(512, 12, 1536, 128, 0) == 0        # invalid k
    assert lib.rd_forward_workspace_size(512, 4096, 1536, 0, 0) == 0        # invalid num_local


def test_unsort_rejects_bad_arguments(lib):
    v = ctypes.c_void_p
    ok = dict(g=16, y=16, w=16, limit=None, grad=16, dot=16, rows=4, hidden=8)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        p = lambda x: None if x is None else v(x)
        return lib.rd_unsort_bwd_rows(p(a["g"]), p(a["y"]), p(a["w"]), p(a["limit"]), p(a["grad"]), p(a["dot"]),
                                      a["rows"], a["hidden"], None)
    assert call(hidden=12) == rd.RD_EUNSUPPORTED
    assert call(hidden=0) == rd.RD_EINVAL
    assert call(rows=-1) == rd.RD_EINVAL
    assert call(g=None) == rd.RD_EINVAL
    assert call(dot=None) == rd.RD_EINVAL
    assert call(grad=24) == rd.RD_EINVAL       # misaligned
    assert call(w=18) == rd.RD_EINVAL          # misaligned float
    assert call(limit=18) == rd.RD_EINVAL      # misaligned int32
    assert call(rows=0, g=None, y=None, w=None, grad=None, dot=None) == rd.RD_OK


def test_zero_rows_from_limit_checks_arguments_before_launch(lib):
    """rd_zero_rows_from_limit: sizes and pointers are checked on the host; the cases that launch
    nothing (no rows, no limit) return OK without touching the GPU."""
    v = ctypes.c_void_p
    ok = dict(buf=16, limit=16, rows=4, row_bytes=32)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        p = lambda x: None if x is None else v(x)
        return lib.rd_zero_rows_from_limit(p(a["buf"]), p(a["limit"]), a["rows"], a["row_bytes"], None)
    assert call(rows=-1) == rd.RD_EINVAL
    assert call(row_bytes=0) == rd.RD_EINVAL
    assert call(row_bytes=-16) == rd.RD_EINVAL
    assert call(row_bytes=24) == rd.RD_EUNSUPPORTED    # not whole 16-byte vectors
    assert call(rows=1 << 40, row_bytes=1 << 30) == rd.RD_EUNSUPPORTED  # rows x row_bytes past 2^62
    assert call(buf=None) == rd.RD_EINVAL
    assert call(buf=24) == rd.RD_EINVAL               # misaligned buffer
    assert call(limit=18) == rd.RD_EINVAL             # misaligned int32
    assert call(rows=0, buf=None, limit=None) == rd.RD_OK
    assert call(limit=None) == rd.RD_OK               # no limit: every row is below it


def test_forward_glu_rejects_bad_arguments(lib):
    """The fused up-projection + GLU: shape rules (k % 64, h % 128) and pointers, checked before launch."""
    v = ctypes.c_void_p
    ok = dict(x=16, w=16, gs=16, G=4, off=None, gl=4, limit=None, act=16, fused=None, m=8, k=64, h=128)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        p = lambda x: None if x is None else v(x)
        return lib.rd_forward_glu(p(a["x"]), p(a["w"]), p(a["gs"]), a["G"], p(a["off"]), a["gl"], p(a["limit"]),
                                  p(a["act"]), p(a["fused"]), a["m"], a["k"], a["h"], None)
    assert call(h=64) == rd.RD_EUNSUPPORTED        # h not a multiple of 128
    assert call(k=72) == rd.RD_EUNSUPPORTED        # k not a multiple of 64
    assert call(k=12) == rd.RD_EUNSUPPORTED        # k not a multiple of 8
    assert call(h=0) == rd.RD_EINVAL
    assert call(act=None) == rd.RD_EINVAL
    assert call(w=None) == rd.RD_EINVAL
    assert call(fused=24) == rd.RD_EINVAL          # misaligned
    assert call(x=40) == rd.RD_EINVAL              # misaligned
    assert call(gl=5, off=16) == rd.RD_EINVAL      # num_local > num_groups
    assert call(m=0, x=None, act=None) == rd.RD_OK  # nothing to do, nothing launched


def test_fp8_forms_reject_bad_sizes(lib):
    """fp8 ragged_dot: k a multiple of 128 for both forms, n a multiple of 16 for the plain form."""
    v = ctypes.c_void_p

    def call(fn, k=128, n=32, m=8):
        return fn(v(16), v(16), v(16), 1, None, 1, None, v(16), 0, m, k, n, None)
    for fn in (lib.rd_forward_fp8, lib.rd_forward_trans_rhs_fp8):
        assert call(fn, k=64) == rd.RD_EUNSUPPORTED
        assert call(fn, k=0) == rd.RD_EINVAL
        assert call(fn, m=0) == rd.RD_OK
    assert call(lib.rd_forward_fp8, n=24) == rd.RD_EUNSUPPORTED


def test_trans_fp8_rejects_bad_arguments(lib):
    """fp8 trans_ragged_dot: k and n multiples of 16, the output dtype, and the row-split workspace
    rules of rd_trans (a size needs a 16-byte aligned pointer), before any launch."""
    v = ctypes.c_void_p

    def call(k=32, n=32, ws=None, ws_bytes=0, dt=0):
        p = lambda x: None if x is None else v(x)
        return lib.rd_trans_fp8(v(16), v(16), v(16), 4, None, 4, None, v(16), dt, 8, k, n, p(ws), ws_bytes, None)
    assert call(k=24) == rd.RD_EUNSUPPORTED
    assert call(n=40) == rd.RD_EUNSUPPORTED
    assert call(dt=7) == rd.RD_EINVAL
    assert call(ws=None, ws_bytes=4096) == rd.RD_EINVAL
    assert call(ws=24, ws_bytes=4096) == rd.RD_EINVAL


def test_tuning_hook_validates_and_restores(lib):
    n = lib.rd_tune_tile_count()
    assert n >= 19
    assert lib.rd_tune_set(rd.RD_TUNE_FWD_TILE, n) == rd.RD_EINVAL
    assert lib.rd_tune_set(rd.RD_TUNE_TRANS_TILE, -2) == rd.RD_EINVAL
    assert lib.rd_tune_set(rd.RD_TUNE_DECODE, 2) == rd.RD_EINVAL
    assert lib.rd_tune_set(7, 0) == rd.RD_EINVAL
    with rd.tuning(fwd_tile=n - 1, trans_tile=0, decode=False):
        pass
    with pytest.raises(rd.RDError):
        with rd.tuning(fwd_tile=n):
            pass
    # the built-in choices are back (no effect is observable without a GPU; the calls succeed)
    assert lib.rd_tune_set(rd.RD_TUNE_FWD_TILE, -1) == rd.RD_OK


def test_noalloc_rejects_sizes_beyond_its_scratch_before_launching(lib):
    # 4096 rows over 256 experts (16 rows each on average), k 4096, n 1536: the decode split path's
    # partial sums need about 96 MiB on a 256-CU device, more than the 80 MiB static scratch
    need = lib.rd_forward_workspace_size(4096, 4096, 1536, 256, 0)
    assert need > rd.RD_NOALLOC_SCRATCH_BYTES
    v = ctypes.c_void_p
    st = lib.rd_forward_noalloc(v(16), v(16), v(16), 256, None, 256, None, v(16), 0, 4096, 4096, 1536, None)
    assert st == rd.RD_ESCRATCH
    assert b"scratch" in lib.rd_status_string(st)
    # the decode step of 64 tokens x top-8 over 128 experts fits
    assert 0 < lib.rd_forward_workspace_size(512, 4096, 1536, 128, 0) <= rd.RD_NOALLOC_SCRATCH_BYTES


# Extreme sizes and counts for the fuzz below (every data pointer NULL, so no call can pass validation
# into a launch: each must return a status, and RD_OK only when there are no rows to process).
_SIZES = [-(1 << 63), -(1 << 31), -1, 0, 1, 7, 8, 16, 24, 64, 136, 4096, (1 << 31) - 1, 1 << 31, 1 << 32,
          (1 << 40) + 8, 1 << 62, (1 << 63) - 1]
_COUNTS = [-(1 << 31), -1, 0, 1, 3, 8, 1024, 1025, (1 << 31) - 1]


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-side fuzz; kept off machines with a GPU")
def test_null_pointer_fuzz_returns_a_status_for_any_sizes(lib):
    """Every entry point with NULL data pointers and sizes drawn from extremes (negative, zero, odd, at and
    past 2^31 / 2^32 / 2^63): a status from the header's list, RD_OK only with nothing to process, and the
    workspace sizes never crash.  (Found a signed overflow of 2 * h in the fused GLU forward's checks.)"""
    rng = np.random.default_rng(7)
    pick = lambda xs: int(xs[rng.integers(len(xs))])
    ok_status = {rd.RD_OK, rd.RD_EINVAL, rd.RD_EUNSUPPORTED}
    # (name, argument kinds, index of the row count): s = int64 size, g = int32 count, d = dtype, w = bytes
    calls = [("rd_forward", "nnngngnndsssnwn", 9), ("rd_forward_trans_rhs", "nnngngnndsssnwn", 9),
             ("rd_forward_noalloc", "nnngngnndsssn", 9), ("rd_forward_fp8", "nnngngnndsssn", 9),
             ("rd_forward_trans_rhs_fp8", "nnngngnndsssn", 9), ("rd_trans", "nnngngnndsssnwn", 9),
             ("rd_trans_fp8", "nnngngnndsssnwn", 9), ("rd_forward_glu", "nnngngnnnsssn", 9),
             ("rd_glu_fwd", "nnnssn", 3), ("rd_glu_bwd", "nnnnssn", 4), ("rd_unsort_bwd_rows", "nnnnnnssn", 6),
             ("rd_zero_rows_from_limit", "nnssn", None)]  # a NULL limit leaves nothing to zero: RD_OK
    for name, kinds, rows_at in calls:
        f = getattr(lib, name)
        for _ in range(600):
            args = []
            for c in kinds:
                if c == "s":
                    args.append(pick(_SIZES))
                elif c == "g":
                    args.append(pick(_COUNTS))
                elif c == "d":
                    args.append(pick([-1, 0, 1, 2, 7]))
                elif c == "w":
                    args.append(pick([0, 1, 256, 1 << 40]))
                else:
                    args.append(None)
            st = f(*args)
            assert st in ok_status, (name, args, st)
            if st == rd.RD_OK and rows_at is not None:
                assert args[rows_at] == 0, (name, args)
    for _ in range(2000):
        m, k, n = pick(_SIZES), pick(_SIZES), pick(_SIZES)
        lib.rd_forward_workspace_size(m, k, n, pick(_COUNTS), pick([0, 1]))
        lib.rd_trans_workspace_size(m, k, n, pick(_COUNTS))


def test_fused_glu_forward_rejects_widths_past_the_limit(lib):
    """h is checked before the weight width 2h is formed."""
    for h, want in ((-5, rd.RD_EINVAL), (0, rd.RD_EINVAL), (1 << 30, rd.RD_EUNSUPPORTED),
                    ((1 << 63) - 1, rd.RD_EUNSUPPORTED)):
        st = lib.rd_forward_glu(None, None, None, 8, None, 8, None, None, None, 64, 128, h, None)
        assert st == want, (h, st)


def test_binding_rejects_operands_on_two_gpus_before_any_call():
    """The binding makes the operands' GPU current for each call; operands (or a stream) on another GPU
    are refused before anything reaches the library."""
    from types import SimpleNamespace
    calls = []
    on0 = SimpleNamespace(device=torch.device("cuda", 0))
    on1 = SimpleNamespace(device=torch.device("cuda", 1))
    with pytest.raises(ValueError, match="one GPU"):
        rd._launch(lambda *a: calls.append(a), (on0, None, on1), None)
    with pytest.raises(ValueError, match="stream on"):
        rd._launch(lambda *a: calls.append(a), (on0, on0), SimpleNamespace(device=torch.device("cuda", 1)))
    assert calls == []

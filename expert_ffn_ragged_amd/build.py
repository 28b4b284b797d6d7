"""Build librd.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Usage: ``python -m expert_ffn_ragged_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles.  Flags: -O3 for gfx950 only; packed-FP32 instructions are
disabled (``-packed-fp32-ops``); no fast-math; the GLU unit additionally
gets ``-ffp-contract=off`` so its float32 op order is exactly the source's.
"""

import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librd.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result",
]
SOURCES = [
    ("rd_gemm.hip", []),
    ("rd_glu.hip", ["-ffp-contract=off"]),
    ("rd_unsort.hip", []),
    ("rd_rows.hip", []),
    ("rd_api.cpp", ["-x", "hip"]),
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("command failed: " + " ".join(shlex.quote(c) for c in cmd))
    return "\n".join(lines)


def build(verbose=False):
    """Compile every source for gfx950 and link librd.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        out = _run([HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

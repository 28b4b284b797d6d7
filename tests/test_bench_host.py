"""Host logic of bench.py, without a GPU: the roofline a kernel is reported
against (HBM below the ridge point, MFMA at or above it) and the refusal of
multi-GPU runs, which the one-GPU benchmark does not measure."""

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_below_the_ridge_is_hbm():
    # the up-projection forward: 137.4 GFLOP over 1.17 GB is 117 flop/B, below the ridge (~315)
    r = bench.roofline("ragged_dot", 0.25, 1.1744e9, 1.3744e11, traffic=1.22e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(1.1744e9 / 0.25e-3 / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS, rel=1e-3)
    assert r["traffic"] == 1220000000


def test_roofline_above_the_ridge_is_mfma():
    ridge = bench.MFMA_BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    nbytes = 1e9
    r = bench.roofline("dx", 0.3, nbytes, 2 * ridge * nbytes)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["traffic"] is None
    assert r["achieved"] == pytest.approx(2 * ridge * nbytes / 0.3e-3 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.MFMA_BF16_PEAK_TFLOPS, rel=1e-3)


def test_zero_flop_kernels_are_hbm():
    r = bench.roofline("glu_fwd", 0.01, 5e7, 0.0)
    assert r["bound"] == "hbm" and r["achieved"] == pytest.approx(5000.0, rel=1e-6)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr

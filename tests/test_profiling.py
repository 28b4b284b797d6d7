"""Host logic of the rocprofv3 summaries (expert_ffn_ragged_amd/profiling.py) on
small synthetic CSV files shaped like rocprofv3's: the calibrated HBM traffic
that bench.py reports, its source-digest guard, the kernel-duration table, the
load-path fractions and the no-host-sync region of an API trace.  No GPU."""

import csv
import os

import pytest

from expert_ffn_ragged_amd import profiling

GEMM = "void rd::(anonymous namespace)::grouped_gemm_stream<0, 128, 512, 3, 32, 1, 1024, 2, 4>(rd::KArgs)"
GLU = "void rd::(anonymous namespace)::glu_fwd_kernel(rd::GluArgs)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def counters(path, rows):
    """rows: (kernel, grid, counter, value)."""
    write_csv(path, ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
              [(k, g, c, v) for k, g, c, v in rows])


def test_short_names_and_ops():
    assert profiling.short_name(GEMM) == "grouped_gemm_stream<0, 128, 512, 3, 32, 1, 1024, 2, 4>"
    assert profiling.op_of(profiling.short_name(GEMM)) == "ragged_dot"
    assert profiling.op_of("glu_bwd_kernel") == "glu_bwd"
    assert profiling.op_of(COPY) is None


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    # the 256 MiB copy reads FETCH_SIZE = 131072 KiB (half its bytes) and writes WRITE_SIZE = 262144 KiB
    counters(tmp_path / "f" / "x_counter_collection.csv", [
        (COPY, 64, "FETCH_SIZE", 1.0),           # a small copy: not the calibration one
        (COPY, 4096, "FETCH_SIZE", 131072.0),
        (GEMM, 256, "FETCH_SIZE", 1000.0),
        (GEMM, 256, "FETCH_SIZE", 3000.0),      # two dispatches: mean 2000 KiB
    ])
    counters(tmp_path / "w" / "x_counter_collection.csv", [
        (COPY, 4096, "WRITE_SIZE", 262144.0),
        (GEMM, 256, "WRITE_SIZE", 500.0),
    ])
    text = profiling.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), None, "cmd")
    row = [ln for ln in text.splitlines() if ln.startswith("| ragged_dot |")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "2"
    read, write, total = float(cells[3]), float(cells[4]), float(cells[5])
    assert read == pytest.approx(2000 * 1024 * 2.0, rel=1e-3)   # fetch counts half the bytes read
    assert write == pytest.approx(500 * 1024, rel=1e-3)
    assert total == pytest.approx(read + write, rel=1e-3)
    out = tmp_path / "traffic.md"
    out.write_text(text)
    assert profiling.load_traffic(str(out))["ragged_dot"] == pytest.approx(total, rel=1e-3)


def test_traffic_is_dropped_once_the_sources_change(tmp_path):
    out = tmp_path / "traffic.md"
    out.write_text("source digest: 0000000000000000\n\n| op | kernel | d | r | w | t |\n"
                   "|---|---|---|---|---|---|\n| ragged_dot | `k` | 1 | 1 | 1 | 2 |\n")
    assert profiling.load_traffic(str(out)) == {}
    assert profiling.load_traffic(str(tmp_path / "missing.md")) == {}


def test_kernel_stats_sorted_by_duration(tmp_path):
    write_csv(tmp_path / "s" / "x_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"], [
        (GLU, 7, 10000.0, 9000.0, 12000.0),
        (GEMM, 7, 300000.0, 250000.0, 330000.0),
        ("some_torch_kernel", 3, 999999.0, 1.0, 2.0),
    ])
    text = profiling.stats_summary(str(tmp_path / "s"), "cmd", "title")
    rows = [ln for ln in text.splitlines() if ln.startswith("| `")]
    assert len(rows) == 2 and "grouped_gemm_stream" in rows[0] and "glu_fwd_kernel" in rows[1]
    assert "| 300.0 |" in rows[0]


def test_load_path_fractions(tmp_path):
    # 8 XCDs x 1000 cycles each; per-CU counters summed over 256 CUs
    counters(tmp_path / "a" / "x_counter_collection.csv", [
        (GEMM, 256, "GRBM_GUI_ACTIVE", 8000.0),
        (GEMM, 256, "TCP_PENDING_STALL_CYCLES", 0.5 * 1000 * 256),
        (GEMM, 256, "TCP_TCC_READ_REQ_LATENCY", 700.0 * 400),
    ])
    counters(tmp_path / "b" / "x_counter_collection.csv", [
        (GEMM, 256, "GRBM_GUI_ACTIVE", 8000.0),
        (GEMM, 256, "TCC_HIT", 100.0),
        (GEMM, 256, "TCC_MISS", 300.0),
    ])
    text = profiling.loadpath_summary([str(tmp_path / "a"), str(tmp_path / "b")], "cmd")
    row = [ln for ln in text.splitlines() if ln.startswith("| ragged_dot |")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "0.50"          # TCP_PENDING_STALL_CYCLES
    assert cells[-2] == "700"          # read latency, cycles per request
    assert cells[-1] == "0.25"         # L2 hit rate


def api_rows(calls):
    return [("HIP_RUNTIME_API", f, 1, 1, cid, t, t + 1) for f, cid, t in calls]


def test_api_region_counts_only_calls_between_the_marks(tmp_path):
    d = tmp_path / "t"
    write_csv(d / "x_hip_api_trace.csv",
              ["Domain", "Function", "Process_Id", "Thread_Id", "Correlation_Id", "Start_Timestamp", "End_Timestamp"],
              api_rows([("hipMalloc", 1, 10), ("hipDeviceSynchronize", 2, 20), ("hipMemGetInfo", 3, 30),
                        ("hipLaunchKernel", 4, 40), ("hipGraphLaunch", 5, 50), ("hipMemGetInfo", 6, 60),
                        ("hipDeviceSynchronize", 7, 70)]))
    write_csv(d / "x_kernel_trace.csv", ["Kernel_Name", "Correlation_Id", "Start_Timestamp"],
              [(GEMM, 4, 1000), (GLU, 5, 1100), (GLU, 1, 5)])
    text = profiling.apitrace_summary(str(d), "cmd")
    assert "Synchronizations, allocations or blocking copies among the calls: **0**" in text
    assert "Memory copies to or from the host: **0**" in text
    assert "| `hipLaunchKernel` | 1 |" in text and "hipMalloc" not in text
    # kernels are matched to the region's calls by correlation id, wherever they ran in time
    assert "| `grouped_gemm_stream<0, 128, 512, 3, 32, 1, 1024, 2, 4>` | 1 |" in text
    assert "| `glu_fwd_kernel` | 1 |" in text


def test_api_region_flags_a_sync_and_a_host_copy(tmp_path):
    d = tmp_path / "t"
    write_csv(d / "x_hip_api_trace.csv",
              ["Domain", "Function", "Process_Id", "Thread_Id", "Correlation_Id", "Start_Timestamp", "End_Timestamp"],
              api_rows([("hipMemGetInfo", 1, 10), ("hipStreamSynchronize", 2, 20), ("hipMemcpyAsync", 3, 25),
                        ("hipMemGetInfo", 4, 30)]))
    write_csv(d / "x_memory_copy_trace.csv", ["Direction", "Correlation_Id", "Start_Timestamp"],
              [("MEMORY_COPY_DEVICE_TO_HOST", 3, 26), ("MEMORY_COPY_DEVICE_TO_HOST", 9, 99)])
    text = profiling.apitrace_summary(str(d), "cmd")
    assert "blocking copies among the calls: **1**" in text
    assert "Memory copies to or from the host: **1**" in text

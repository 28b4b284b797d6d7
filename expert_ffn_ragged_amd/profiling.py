"""Summaries of rocprofv3 output for the ragged-dot kernels, and their lookup.

Turns the CSV files of ``rocprofv3 --kernel-trace --stats`` and of
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` / MFMA-counter runs of
``bench.py`` into short Markdown summaries (kept under ``profiles/``), and
reads the HBM traffic back for ``bench.py``'s roofline.

HBM bytes: ``FETCH_SIZE`` and ``WRITE_SIZE`` (KiB per dispatch, summed over
the L2 channels) are scaled by what the same counter reads for a plain copy
kernel of known size (``bench.py --copy-calib`` copies 256 MiB), so that the
reported bytes are calibrated against an operation whose traffic is known.
A summary records a digest of the kernel sources; ``bench.py`` reports the
traffic only while the digest still matches (the kernels have not changed
since the counters were taken).

Usage (on the host, after copying the rocprofv3 output directories back)::

    python -m expert_ffn_ragged_amd.profiling traffic --fetch DIR --write DIR \\
        [--mfma DIR] --command "..." --out profiles/upproj_fwd_bwd_traffic.md
    python -m expert_ffn_ragged_amd.profiling stats --stats DIR --command "..." --out FILE.md
    python -m expert_ffn_ragged_amd.profiling apitrace --trace DIR --command "..." --out FILE.md
"""

import argparse
import csv
import glob
import hashlib
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CALIB_BYTES = 256 << 20  # the calibration copy of bench.py --copy-calib
SIMDS = 1024             # 256 CUs x 4 SIMDs
XCDS = 8

# bench.py op name <- kernel name pattern (one kernel per op in the step)
OP_OF_KERNEL = (
    (r"grouped_gemm_(stream|pp|regs)<0,", "ragged_dot"),
    (r"grouped_gemm_(stream|pp|regs)<1,", "ragged_dot_trans_rhs"),
    (r"grouped_gemm_(stream|pp|regs)<2,", "trans_ragged_dot"),
    (r"grouped_gemm_(stream|pp)<4,", "ragged_dot_glu"),
    (r"unsort_bwd_rows_kernel", "unsort_bwd_rows"),
    (r"zero_rows_kernel", "zero_rows_from_limit"),
    (r"glu_fwd_kernel", "glu_fwd"),
    (r"glu_bwd_kernel", "glu_bwd"),
    (r"decode_streamk_gemm", "decode_gemm"),
    (r"decode_streamk_reduce", "decode_reduce"),
    (r"trans_split_reduce", "trans_split_reduce"),
)


def source_digest():
    """sha256 (16 hex digits) of the kernel sources and the C header."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + [os.path.join(ROOT, "include", "rd.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(kernel):
    k = kernel.replace("void ", "").replace("rd::(anonymous namespace)::", "")
    k = re.sub(r"\(rd::KArgs\)|\(KArgs.*", "", k)
    return re.sub(r"\(.*", "", k).strip()


def op_of(kernel):
    for pat, op in OP_OF_KERNEL:
        if re.search(pat, kernel):
            return op
    return None


def _rows(directory, suffix):
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def counter_means(directory):
    """{(kernel short name, counter): (mean value, dispatches)} over a counter_collection CSV."""
    acc = {}
    calib = {}
    for row in _rows(directory, "counter_collection.csv"):
        name, ctr, val = row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])
        if "copyBuffer" in name:
            calib.setdefault(ctr, []).append((int(row["Grid_Size"]), val))
            continue
        if op_of(name) is None:
            continue
        acc.setdefault((short_name(name), ctr), []).append(val)
    means = {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}
    # the calibration copy is the largest copyBuffer dispatch
    cal = {}
    for ctr, vals in calib.items():
        big = max(g for g, _ in vals)
        sel = [v for g, v in vals if g == big]
        cal[ctr] = sum(sel) / len(sel)
    return means, cal


DEFAULT_TITLE = "MoE up-projection fwd+bwd step (m8192 k4096 n2048 g64 Zipf 1.1), MI355X"


def traffic_summary(fetch_dir, write_dir, mfma_dir, command, title=DEFAULT_TITLE):
    fm, fcal = counter_means(fetch_dir)
    wm, wcal = counter_means(write_dir)
    fscale = CALIB_BYTES / (fcal["FETCH_SIZE"] * 1024)
    wscale = CALIB_BYTES / (wcal["WRITE_SIZE"] * 1024)
    lines = [
        f"# HBM traffic per launch: {title}",
        "",
        "Commands (run from the repository root on the GPU box with `TMPDIR=/tmp` exported; one counter",
        "per run, each run its own process):",
        "",
        "```",
        command,
        "```",
        "",
        f"Calibration: a 256 MiB device-to-device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = "
        f"{fcal['FETCH_SIZE']:.0f} KiB and WRITE_SIZE = {wcal['WRITE_SIZE']:.0f} KiB, so bytes = "
        f"FETCH_SIZE x 1024 x {fscale:.4f} and WRITE_SIZE x 1024 x {wscale:.4f}.",
        "",
        f"source digest: {source_digest()}",
        "",
        "| op | kernel | dispatches | read (bytes) | write (bytes) | traffic (bytes) |",
        "|---|---|---|---|---|---|",
    ]
    for (name, ctr), (val, n) in sorted(fm.items()):
        if ctr != "FETCH_SIZE":
            continue
        w = wm.get((name, "WRITE_SIZE"), (0.0, 0))[0]
        rb, wb = val * 1024 * fscale, w * 1024 * wscale
        lines.append(f"| {op_of(name)} | `{name}` | {n} | {rb:.4g} | {wb:.4g} | {rb + wb:.4g} |")
    if mfma_dir:
        mm, _ = counter_means(mfma_dir)
        lines += ["", "MFMA counters (same command with `--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                  "GRBM_GUI_ACTIVE SQ_BUSY_CYCLES`). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                  f"(GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs); MFMA flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.",
                  "", "| op | kernel | MFMA busy | MFMA flop per launch |", "|---|---|---|---|"]
        names = sorted({n for n, c in mm if c == "SQ_VALU_MFMA_BUSY_CYCLES"})
        for name in names:
            busy = mm[(name, "SQ_VALU_MFMA_BUSY_CYCLES")][0]
            gui = mm[(name, "GRBM_GUI_ACTIVE")][0]
            mops = mm.get((name, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), (0.0, 0))[0]
            util = busy / (gui / XCDS * SIMDS) if gui else 0.0
            lines.append(f"| {op_of(name)} | `{name}` | {util:.3f} | {mops * 512:.4g} |")
    return "\n".join(lines) + "\n"


def steady_durations(stats_dir, skip):
    """{kernel short name: [durations in us]} from the kernel trace, dropping each kernel's first `skip`
    dispatches (the warm-up launches of the profiled command)."""
    per = {}
    for row in sorted(_rows(stats_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        if op_of(row["Kernel_Name"]) is None:
            continue
        per.setdefault(short_name(row["Kernel_Name"]), []).append(
            (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    return {k: v[skip:] for k, v in per.items() if len(v) > skip}


def stats_summary(stats_dir, command, title, skip=0):
    rows = []
    for row in _rows(stats_dir, "kernel_stats.csv"):
        if op_of(row["Name"]) is None:
            continue
        rows.append((short_name(row["Name"]), int(row["Calls"]), float(row["AverageNs"]) / 1e3,
                     float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3))
    steady = steady_durations(stats_dir, skip) if skip else {}
    lines = [f"# Kernel durations: {title}", "", "Command (run from the repository root on the GPU box "
             "with `TMPDIR=/tmp` exported):", "", "```", command, "```", "",
             f"source digest: {source_digest()}", ""]
    if skip:
        lines += [f"The last two columns leave out each kernel's first {skip} dispatches (the command's untimed "
                  "settle and warm-up launches), from the kernel trace of the same run.", ""]
    lines += ["| kernel | calls | average (us) | min (us) | max (us) |" + (" timed calls | timed average (us) |"
                                                                          if skip else ""),
              "|---|---|---|---|---|" + ("---|---|" if skip else "")]
    for name, calls, avg, mn, mx in sorted(rows, key=lambda r: -r[2]):
        extra = ""
        if skip:
            d = steady.get(name, [])
            extra = f" {len(d)} | {sum(d) / len(d):.1f} |" if d else " 0 | - |"
        lines.append(f"| `{name}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} |" + extra)
    return "\n".join(lines) + "\n"


# HIP API calls that would break the no-host-sync property inside the marked region
# (copies are judged by the memory-copy trace's direction: a device-to-device rewrite is allowed)
SYNC_CALLS = re.compile(r"Synchronize|Malloc|Free|DtoH|Query|hipMemcpy$|WithStream")


def apitrace_summary(trace_dir, command):
    """HIP API calls, memory copies and kernels between the two hipMemGetInfo marks of
    ``bench.py --api-region``, from a ``rocprofv3 --hip-trace --memory-copy-trace --kernel-trace`` run."""
    api = list(_rows(trace_dir, "hip_api_trace.csv"))
    marks = sorted(int(r["Start_Timestamp"]) for r in api if r["Function"] == "hipMemGetInfo")
    if len(marks) < 2:
        raise SystemExit("no pair of hipMemGetInfo marks in the trace")
    t0, t1 = marks[-2], marks[-1]
    inside = [r for r in api if t0 < int(r["Start_Timestamp"]) < t1]
    calls = {}
    for r in inside:
        calls[r["Function"]] = calls.get(r["Function"], 0) + 1
    copies = {}
    for r in _rows(trace_dir, "memory_copy_trace.csv"):
        if t0 < int(r["Start_Timestamp"]) < t1:
            key = r.get("Direction") or r.get("Kind") or "copy"
            copies[key] = copies.get(key, 0) + 1
    # kernels dispatched by the region's calls (matched by correlation id; they may run after the mark)
    ids = {r["Correlation_Id"] for r in inside}
    kernels = {}
    for r in _rows(trace_dir, "kernel_trace.csv"):
        if r["Correlation_Id"] in ids:
            name = short_name(r["Kernel_Name"])
            kernels[name] = kernels.get(name, 0) + 1
    bad = {f: c for f, c in calls.items() if SYNC_CALLS.search(f)}
    to_host = {k: c for k, c in copies.items() if "HOST" in k.upper()}
    lines = ["# HIP API trace of the library's calls: decode layer (eager and graph replays) and the "
             "up-projection fwd+bwd step, MI355X", "",
             "Command (run from the repository root on the GPU box with `TMPDIR=/tmp` exported):", "",
             "```", command, "```", "",
             "The region lies between the two `hipMemGetInfo` marks of `bench.py --api-region`: five rounds of "
             "the decode layer (ragged_dot then GLU, eagerly), a device-to-device rewrite of group_sizes, a "
             "replay of the same layer captured as a graph, and the five kernels of the up-projection step.", "",
             f"source digest: {source_digest()}", "",
             f"Synchronizations, allocations or blocking copies among the calls: **{sum(bad.values())}**"
             + (f" ({bad})" if bad else "") + ".",
             f"Memory copies to or from the host: **{sum(to_host.values())}**"
             + (f" ({to_host})" if to_host else "") + ".", "",
             "| HIP API call | calls in the region |", "|---|---|"]
    for f, c in sorted(calls.items(), key=lambda kv: -kv[1]):
        lines.append(f"| `{f}` | {c} |")
    lines += ["", "| memory copy | count |", "|---|---|"]
    for k, c in sorted(copies.items()):
        lines.append(f"| {k} | {c} |")
    if not copies:
        lines.append("| none recorded (the group_sizes rewrites are copy kernels on the device) | 0 |")
    lines += ["", "| kernel | dispatches by the region's calls |", "|---|---|"]
    for k, c in sorted(kernels.items(), key=lambda kv: -kv[1]):
        lines.append(f"| `{k}` | {c} |")
    return "\n".join(lines) + "\n"


# per-instance counters (one instance per CU) reported as a fraction of the kernel's cycles
PER_CU = ("TCP_PENDING_STALL_CYCLES", "TCP_UTCL1_STALL_INFLIGHT_MAX", "TA_TA_BUSY", "TA_ADDR_STALLED_BY_TC_CYCLES",
          "TD_TD_BUSY", "TD_TC_STALL")
CUS = 256


def loadpath_summary(dirs, command, title=DEFAULT_TITLE):
    """Load-path counters of the step's kernels: per-CU busy / stall fractions (counter summed over the
    256 CUs / (GRBM_GUI_ACTIVE / 8 XCDs x 256)), the mean L1 -> L2 read latency
    (TCP_TCC_READ_REQ_LATENCY / (TCC_HIT + TCC_MISS)) and the L2 hit rate."""
    means = {}
    for d in dirs:
        m, _ = counter_means(d)
        for (name, ctr), (val, _n) in m.items():
            means.setdefault(name, {}).setdefault(ctr, []).append(val)
    lines = [f"# Load-path counters: {title}", "",
             "Commands (run from the repository root on the GPU box with `TMPDIR=/tmp` exported; one counter set "
             "per run):", "", "```", command, "```", "",
             f"source digest: {source_digest()}", "",
             "Per-CU fractions are the counter summed over the 256 CUs divided by the kernel's cycles "
             "(GRBM_GUI_ACTIVE / 8 XCDs) x 256. Read latency is TCP_TCC_READ_REQ_LATENCY / (TCC_HIT + TCC_MISS), "
             "in cycles per L1 -> L2 read request.", "",
             "| op | kernel | " + " | ".join(PER_CU) + " | read latency (cycles) | L2 hit rate |",
             "|---|---|" + "---|" * (len(PER_CU) + 2)]
    readings = []
    for name, ctrs in sorted(means.items(), key=lambda kv: str(op_of(kv[0]))):
        if op_of(name) is None or "GRBM_GUI_ACTIVE" not in ctrs:
            continue
        gui = sum(ctrs["GRBM_GUI_ACTIVE"]) / len(ctrs["GRBM_GUI_ACTIVE"]) / XCDS

        def frac(c):
            return f"{ctrs[c][0] / (gui * CUS):.2f}" if c in ctrs and gui else "-"

        req = (ctrs.get("TCC_HIT", [0])[0] + ctrs.get("TCC_MISS", [0])[0])
        lat = f"{ctrs['TCP_TCC_READ_REQ_LATENCY'][0] / req:.0f}" if req and "TCP_TCC_READ_REQ_LATENCY" in ctrs else "-"
        hit = f"{ctrs['TCC_HIT'][0] / req:.2f}" if req and "TCC_HIT" in ctrs else "-"
        lines.append(f"| {op_of(name)} | `{name}` | " + " | ".join(frac(c) for c in PER_CU) + f" | {lat} | {hit} |")
        if "grouped_gemm" in name and all(c in ctrs for c in ("TCP_PENDING_STALL_CYCLES", "TD_TD_BUSY", "TD_TC_STALL")):
            readings.append(
                f"- {op_of(name)}: the vector L1 of each CU waits on data pending from L2 "
                f"{100 * float(frac('TCP_PENDING_STALL_CYCLES')):.0f} % of its cycles. The data-return unit is "
                f"{100 * float(frac('TD_TD_BUSY')):.0f} % busy, "
                f"{100 * float(frac('TD_TC_STALL')):.0f} % of the cycles stalled on the cache. The L2 hit rate is "
                f"{hit}, and {lat} cycles is the mean read latency.")
    if readings:
        lines += ["", "What caps the grouped GEMMs: the load stream into each CU, not the MFMAs. A stage is "
                  "complete only when its slowest line has arrived, so the lines that miss L2 hold up each stage.",
                  ""] + readings
    return "\n".join(lines) + "\n"


def load_traffic(path):
    """{op: traffic bytes per launch} from a traffic summary whose digest matches the sources, else {}."""
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        text = f.read()
    m = re.search(r"^source digest: (\w+)", text, flags=re.M)
    if not m or m.group(1) != source_digest():
        return {}
    out = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0] not in ("op", "---"):
            try:
                out[cells[0]] = float(cells[5])
            except ValueError:
                pass
    return out


def main():
    ap = argparse.ArgumentParser(description="summaries of rocprofv3 output for the ragged-dot kernels")
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--mfma")
    t.add_argument("--title", default=DEFAULT_TITLE)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--stats", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--skip", type=int, default=0, help="leave out each kernel's first N dispatches")
    s.add_argument("--out", required=True)
    lp = sub.add_parser("loadpath")
    lp.add_argument("--dirs", nargs="+", required=True)
    lp.add_argument("--title", default=DEFAULT_TITLE)
    lp.add_argument("--command", required=True)
    lp.add_argument("--out", required=True)
    r = sub.add_parser("apitrace")
    r.add_argument("--trace", required=True)
    r.add_argument("--command", required=True)
    r.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "traffic":
        text = traffic_summary(a.fetch, a.write, a.mfma, a.command, a.title)
    elif a.what == "loadpath":
        text = loadpath_summary(a.dirs, a.command, a.title)
    elif a.what == "apitrace":
        text = apitrace_summary(a.trace, a.command)
    else:
        text = stats_summary(a.stats, a.command, a.title, a.skip)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()

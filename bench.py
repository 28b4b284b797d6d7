"""Benchmark of the ragged-dot hot path on one MI355X.

Headline step: the MoE backward of a down-projection, the one shape of the
path that sits at the MFMA ridge (2 x 274.9 GFLOP on 1.7 GB): 32768 rows,
64 experts with Zipf(1.1) sizes (4 of them empty), w [64, 1024, 4096] bf16:

    dx = ragged_dot(dy [32768, 4096], w, gs, trans_rhs)   [32768, 1024] bf16
    dW = trans_ragged_dot(x [32768, 1024], dy, gs)         [64, 1024, 4096] bf16

``value`` is the GEMM work on valid rows (2 x 2 * sum(gs) * 1024 * 4096
FLOP) per second of step time, cold: L2 and the 256 MB MALL are flushed
before every timed step (a 512 MiB write outside the events), inputs
resident in HBM.  Each step is bracketed by HIP events on the stream the
kernels run on, with one more event between dx and dW, which gives each
kernel's time; the slower kernel is reported against its roofline.  The
same step is also timed warm (steps back to back, events only at the ends).
Before the first timed loop the step runs untimed, cold, SETTLE_STEPS
times, so the timed loops see the steady state of repeated steps.
The other workloads (up-projection forward+backward, decode, window+limit,
GLU and unsort over the packed buffer, fp8) are reported under ``extra``.
Inputs are synthetic and seeded (expert_ffn_ragged_amd/workloads.py).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (no sparsity)
MFMA_FP8_PEAK_TFLOPS = 5033.2  # MI355X dense fp8 MFMA, published (no sparsity)
# the hot expert's rows (of 32768) for the split / unsplit comparison beyond the default 60 %
HOT_SHARES = (("80", 26214), ("95", 31130))
METRIC = "ragged_dot TFLOP/s (valid rows) + % bf16 MFMA peak; decode-shape HBM GB/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--all", action="store_true",
                    help="also time the window+limit, packed-buffer GLU and unsort, fp8 and MoE MLP workloads")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline step (for profiler runs), no extra workloads")
    ap.add_argument("--sweep", action="store_true",
                    help="time every tile shape of every grouped GEMM on the workloads and print the table")
    ap.add_argument("--profile", choices=("backward", "upproj", "decode", "packed"),
                    help="only run one workload's kernels, --warmup + --steps times each, for a profiler")
    ap.add_argument("--settle", type=int, default=0,
                    help="with --profile: untimed passes before the warmup, flushed with --cold (the headline "
                         f"settles for {SETTLE_STEPS} cold steps)")
    ap.add_argument("--cold", action="store_true",
                    help="with --profile: flush L2 and the MALL (a 512 MiB write) before every pass")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first copy 256 MiB device-to-device three times (reference kernel for HBM counters)")
    ap.add_argument("--api-region", action="store_true",
                    help="only run the marked region for a HIP API trace (see api_region) and exit")
    return ap.parse_args()


PERCENTILES = {}  # op -> (p10, p50, p90) in ms, filled by timed_ops
COLD = {"on": False, "buf": None}


def flush_caches():
    """Write a 512 MiB scratch buffer: evicts L2 and the 256 MB MALL before a cold iteration."""
    import torch

    if COLD["buf"] is None:
        COLD["buf"] = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    COLD["buf"].fill_(1)


def timed_ops(ops, steps, warmup):
    """Run `warmup` untimed steps, then `steps` timed ones with per-op HIP events on the current stream.

    With COLD on, the caches are flushed before every timed step, outside the events.
    Returns (wall seconds, GPU ms from the first to the last event, {op: mean ms}); the
    per-op p10/p50/p90 go to PERCENTILES.
    """
    import torch

    for _ in range(warmup):
        for _, fn in ops:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
           for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        if COLD["on"]:
            flush_caches()
        for (_, fn), (a, b) in zip(ops, evs[s]):
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = {}
    for i, (name, _) in enumerate(ops):
        t = sorted(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(steps))
        per_op[name] = sum(t) / steps
        q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
        PERCENTILES[name] = (round(q(0.1), 4), round(q(0.5), 4), round(q(0.9), 4))
    first, last = evs[0][0][0], evs[-1][-1][1]
    gpu_ms = first.elapsed_time(last)
    if COLD["on"]:  # the flushes sit between the events: the step is the sum of its ops
        gpu_ms = sum(per_op.values()) * steps
    return wall, gpu_ms, per_op


SETTLE_STEPS = 300  # untimed cold steps before the first timed loop of a process (about 0.25 s)


def settle(ops, steps=SETTLE_STEPS, cold=True):
    """Run the ops untimed `steps` times, each after a cache flush when cold (synchronizing every 50),
    so the timed loops see the steady state of repeated steps.  Measured on the backward: the first
    cold loop of a process (5 warm-up + 20 timed steps) took 0.80 ms a step, every later one 0.70-0.72;
    1500 warm steps before it, or 300 flushes alone, left it at 0.77; 300 cold steps removed it."""
    import torch

    for i in range(steps):
        if cold:
            flush_caches()
        for _, fn in ops:
            fn()
        if i % 50 == 49:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return steps


def step_timed(ops, steps, warmup):
    """GPU ms of `steps` back-to-back eager steps with events only around the whole run (the per-op
    events of timed_ops add their own dispatch overhead between kernels)."""
    import torch

    for _ in range(warmup):
        for _, fn in ops:
            fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        for _, fn in ops:
            fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def upproj(steps, warmup):
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    d = workloads.make(2, "cuda", parts=("x", "w"))
    x, w, gs = d["x"], d["w"], d["gs"]
    m, k, n = d["m"], d["k"], d["n"]
    rows = int(d["gs_host"].sum())
    d_act = workloads.bf16_normal((m, n // 2), 1.0, 2006, "cuda")
    fused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((m, n // 2), dtype=torch.bfloat16, device="cuda")
    dfused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((w.shape[0], k, n), dtype=torch.bfloat16, device="cuda")
    ops = [
        ("ragged_dot", lambda: rd.ragged_dot(x, w, gs, out=fused)),
        ("glu_fwd", lambda: rd.glu_fwd(fused, out=act)),
        ("glu_bwd", lambda: rd.glu_bwd(fused, d_act, out=dfused)),
        ("ragged_dot_trans_rhs", lambda: rd.ragged_dot(dfused, w, gs, trans_rhs=True, out=dx)),
        ("trans_ragged_dot", lambda: rd.trans_ragged_dot(x, dfused, gs, out=dw)),
    ]
    wall, gpu_ms, per_op = timed_ops(ops, steps, warmup)
    # the headline step: the same launches with no events between them (warm mode; the cold mode's
    # flushes sit between steps, so there the step is the sum of its timed ops)
    step_ms = None if COLD["on"] else step_timed(ops, steps, warmup)
    gemm_flop = 2.0 * rows * k * n
    b = 2  # bf16 bytes
    # algorithmic bytes: every operand read once, every result written once
    nbytes = {
        "ragged_dot": rows * k * b + w.numel() * b + rows * n * b,
        "ragged_dot_trans_rhs": rows * n * b + w.numel() * b + rows * k * b,
        "trans_ragged_dot": rows * k * b + rows * n * b + w.numel() * b,
        "glu_fwd": rows * n * b + rows * (n // 2) * b,
        "glu_bwd": rows * n * b + rows * (n // 2) * b + rows * n * b,
    }
    flops = {"ragged_dot": gemm_flop, "ragged_dot_trans_rhs": gemm_flop, "trans_ragged_dot": gemm_flop,
             "glu_fwd": 0.0, "glu_bwd": 0.0}
    return dict(rows=rows, m=m, k=k, n=n, G=w.shape[0], wall=wall, gpu_ms=gpu_ms, step_ms=step_ms, per_op=per_op,
                bytes=nbytes, flops=flops, step_flop=3 * gemm_flop,
                tensors=(x, w, dfused, d["gs_host"]))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "upproj_fwd_bwd_traffic.md")
BACKWARD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "backward_m32768_traffic.md")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_m512_traffic.md")
PACKED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "packed_buffer_limit126156_traffic.md")


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch from a committed counter summary, while the kernels are unchanged."""
    from expert_ffn_ragged_amd import profiling

    return profiling.load_traffic(path)


BACKWARD_WORKLOAD = ("moe backward m32768: dx = ragged_dot(dy[32768,4096], w[64,1024,4096], trans_rhs) + "
                     "dW = trans_ragged_dot(x[32768,1024], dy) bf16, g64 zipf1.1, 4 empty groups")


def backward(steps, warmup):
    """The headline step, cold (caches flushed before each step) and warm."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    d = workloads.make(3, "cuda")
    x, w, dy, gs = d["x"], d["w"], d["dy"], d["gs"]
    m, k, n = d["m"], d["k"], d["n"]  # x [m, k], dy [m, n], w [G, k, n] (k = n_out of dx)
    rows = int(d["gs_host"].sum())
    nonempty = int((d["gs_host"] > 0).sum())
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((d["G"], k, n), dtype=torch.bfloat16, device="cuda")
    ops = [
        ("ragged_dot_trans_rhs", lambda: rd.ragged_dot(dy, w, gs, trans_rhs=True, out=dx)),
        ("trans_ragged_dot", lambda: rd.trans_ragged_dot(x, dy, gs, out=dw)),
    ]
    settled = settle(ops)
    COLD["on"] = True
    wall, cold_ms, cold_per = timed_ops(ops, steps, warmup)
    cold_pct = {name: PERCENTILES[name] for name, _ in ops}
    COLD["on"] = False
    _, _, warm_per = timed_ops(ops, steps, warmup)
    warm_step = step_timed(ops, steps, warmup) / steps
    flop = 2.0 * rows * k * n
    b = 2  # bf16 bytes
    # algorithmic bytes: every operand read once (the weights of non-empty experts only), every result
    # written once (dW of an empty expert is written as zeros)
    nbytes = {"ragged_dot_trans_rhs": rows * n * b + nonempty * k * n * b + rows * k * b,
              "trans_ragged_dot": rows * k * b + rows * n * b + d["G"] * k * n * b}
    return dict(rows=rows, m=m, k=k, n=n, G=d["G"], wall=wall, settle_steps=settled, cold_ms=cold_ms / steps,
                cold_per=cold_per,
                cold_pct=cold_pct, warm_per=warm_per, warm_step=warm_step, bytes=nbytes,
                flops={"ragged_dot_trans_rhs": flop, "trans_ragged_dot": flop}, step_flop=2 * flop,
                tensors=(x, w, dy, d["gs_host"]))


def roofline(name, ms, nbytes, flop, traffic=None):
    """Report a kernel against the roof its arithmetic intensity puts it under."""
    ai = flop / nbytes if nbytes else 0.0
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    t = None if traffic is None else int(traffic)
    if flop > 0 and ai >= ridge:
        achieved = flop / (ms * 1e-3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": t,
                "ms": round(ms, 4), "algorithmic_bytes": int(nbytes), "flop": flop}
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": t, "ms": round(ms, 4),
            "algorithmic_bytes": int(nbytes), "flop": flop}


def extra_workloads(steps, warmup):
    """The up-projection forward+backward step and the decode GEMM (reported beside the headline)."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    out = {}
    r = upproj(steps, warmup)
    traffic = measured_traffic()
    step_ms = r["step_ms"] / steps
    out["upproj_fwd_bwd_m8192_k4096_n2048_g64"] = {
        "ms_per_step": round(step_ms, 4), "TFLOP/s": round(r["step_flop"] / step_ms / 1e9, 1),
        "mfma_frac": round(r["step_flop"] / step_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
        "timing": "warm; steps back to back, per-kernel times from a loop with events around each launch",
        "per_kernel": {name: dict(roofline(name, ms, r["bytes"][name], r["flops"][name], traffic.get(name)),
                                  p10_p50_p90_ms=PERCENTILES.get(name))
                       for name, ms in r["per_op"].items()}}
    del r
    torch.cuda.empty_cache()
    d = workloads.make(5, "cuda", parts=("x", "w"))
    o = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device="cuda")
    wsb = rd.library().rd_forward_workspace_size(d["m"], d["k"], d["n"], d["G"], 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    _, _, per = timed_ops([("decode", lambda: rd.ragged_dot(d["x"], d["w"], d["gs"], out=o, workspace=ws))],
                          steps, warmup)
    nz = d["gs_host"] > 0
    rows = int(d["gs_host"].sum())
    # algorithmic bytes: x rows, the weights of non-empty experts, the output
    nb = rows * d["k"] * 2 + int(nz.sum()) * d["k"] * d["n"] * 2 + rows * d["n"] * 2
    tr = measured_traffic(DECODE_TRAFFIC_FILE)
    t = (tr["decode_gemm"] + tr.get("decode_reduce", 0.0)) if "decode_gemm" in tr else None
    out["decode_m512_k4096_n1536_g128"] = {
        "ms": round(per["decode"], 4), "GB/s": round(nb / per["decode"] / 1e6, 1),
        "hbm_frac": round(nb / per["decode"] / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(nb),
        "traffic": None if t is None else int(t), "p10_p50_p90_ms": PERCENTILES.get("decode")}
    out["decode_layer_graph_m512"] = decode_graph(d, ws, steps, warmup)
    del d, o
    torch.cuda.empty_cache()
    return out


def decode_graph(d, ws, steps, warmup):
    """The decode layer (wi ragged_dot, GLU, wo ragged_dot, one device-resident group_sizes; wo is
    [128, 768, 4096]) captured as one graph and replayed; between replays a device-side copy rewrites
    group_sizes (alternating two size vectors), outside the events.  After the timed replays, the last
    replay's output is checked bit for bit against the same layer run eagerly on the same sizes."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    m, n = d["m"], d["n"]
    h, d_out = n // 2, 4096
    gs_a, gs_b = d["gs"].clone(), torch.roll(d["gs"], 1).contiguous()
    gs = gs_a.clone()
    o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((m, h), dtype=torch.bfloat16, device="cuda")
    wo = workloads.bf16_normal((d["G"], h, d_out), 0.02, 2009, "cuda")
    out = torch.empty((m, d_out), dtype=torch.bfloat16, device="cuda")
    ws2 = torch.empty(max(rd.library().rd_forward_workspace_size(m, h, d_out, d["G"], 0), 16), dtype=torch.uint8,
                      device="cuda")

    def layer():
        rd.ragged_dot(d["x"], d["w"], gs, out=o, workspace=ws)
        rd.glu_fwd(o, out=act)
        rd.ragged_dot(act, wo, gs, out=out, workspace=ws2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        layer()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(warmup + steps):
        gs.copy_(gs_b if i % 2 else gs_a)  # device-side rewrite, outside the events
        if i >= warmup:
            evs[i - warmup][0].record(stream)
        graph.replay()
        if i >= warmup:
            evs[i - warmup][1].record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    got = out.clone()
    last = gs_b if (warmup + steps - 1) % 2 else gs_a
    gs.copy_(last)
    layer()
    torch.cuda.synchronize()
    if not torch.equal(got.view(torch.int16), out.view(torch.int16)):
        raise RuntimeError("decode graph replay differs from the eager layer")
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    ms = sum(t) / len(t)
    # algorithmic bytes of the replays' two size vectors (averaged): x, the weights of non-empty experts of
    # wi and wo, the [gate | up] buffer written and read, act written and read, the output
    nb = 0
    for g in (gs_a, gs_b):
        sz = g.cpu().numpy()
        rows, nz = int(sz.sum()), int((sz > 0).sum())
        nb += (rows * d["k"] * 2 + nz * d["k"] * n * 2 + 2 * rows * n * 2 + 2 * rows * h * 2 + nz * h * d_out * 2
               + rows * d_out * 2) / 2
    return {"ms": round(ms, 4), "p10_p50_p90_ms": [round(q(0.1), 4), round(q(0.5), 4), round(q(0.9), 4)],
            "GB/s": round(nb / ms / 1e6, 1), "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4),
            "timing": "replays of one captured graph (wi ragged_dot -> GLU -> wo ragged_dot), group_sizes "
                      "rewritten on the device between replays (outside the events); last replay checked "
                      "bitwise against eager"}


def extra_all(steps):
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    out = {}
    d = workloads.make(3, "cuda")
    gs3 = d["gs"]
    m, k, n = d["m"], d["k"], d["n"]
    rows = int(d["gs_host"].sum())
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((d["G"], k, n), dtype=torch.bfloat16, device="cuda")
    dw32 = torch.empty((d["G"], k, n), dtype=torch.float32, device="cuda")
    _, _, per = timed_ops([
        ("dw_f32", lambda: rd.trans_ragged_dot(d["x"], d["dy"], d["gs"], out=dw32)),
    ], steps, 3)
    # context: the vendor library's dense bf16 GEMM of the same flops (dy [m, n] times one expert's
    # w [k, n] transposed, no grouping), through torch
    wd = d["w"][0].contiguous()
    _, _, per_d = timed_ops([("dense", lambda: torch.nn.functional.linear(d["dy"], wd))], steps, 3)
    fl = 2.0 * rows * k * n
    for key, ms in per.items():
        out[f"backward_m32768_{key}"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                        "mfma_frac": round(fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # one hot expert (60 % of the rows) at the same shape: trans_ragged_dot with the row split of long
    # groups (the default) and without it
    gsh = torch.tensor(workloads.hot_expert_sizes(), dtype=torch.int32, device="cuda")
    _, _, per_h = timed_ops([
        ("split", lambda: rd.trans_ragged_dot(d["x"], d["dy"], gsh, out=dw)),
        ("unsplit", lambda: rd.trans_ragged_dot(d["x"], d["dy"], gsh, out=dw, row_split=False)),
    ], steps, 3)
    out["backward_m32768_hot_expert_dw"] = {
        key: {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1)} for key, ms in per_h.items()}
    out["backward_m32768_hot_expert_dw"]["sizes"] = "19660 rows in one expert, the rest Zipf(1.1) over 63"
    # the same with 80 % and 95 % of the rows in the hot expert, split / unsplit (fp8 below)
    shares = {"60": {key: round(ms, 4) for key, ms in per_h.items()}}
    for pct, hot_rows in HOT_SHARES:
        gsx = torch.tensor(workloads.hot_expert_sizes(hot_rows=hot_rows), dtype=torch.int32, device="cuda")
        _, _, per_x = timed_ops([
            ("split", lambda: rd.trans_ragged_dot(d["x"], d["dy"], gsx, out=dw)),
            ("unsplit", lambda: rd.trans_ragged_dot(d["x"], d["dy"], gsx, out=dw, row_split=False)),
        ], steps, 3)
        shares[pct] = {key: round(ms, 4) for key, ms in per_x.items()}
    hot_shares = {"unit": "ms", "rows_in_hot_expert": {"60": 19660, **{p: r for p, r in HOT_SHARES}},
                  "bf16": shares}
    fld = 2.0 * m * k * n
    out["backward_m32768_dx_dense_torch_reference"] = {
        "ms": round(per_d["dense"], 4), "TFLOP/s": round(fld / per_d["dense"] / 1e9, 1),
        "mfma_frac": round(fld / per_d["dense"] / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del wd
    # the same dx with fp8 (E4M3) operands
    dy8, w8, x8 = d["dy"].to(torch.float8_e4m3fn), d["w"].to(torch.float8_e4m3fn), d["x"].to(torch.float8_e4m3fn)
    del d, dw, dw32
    torch.cuda.empty_cache()
    out.update(glu_epilogue(steps))
    _, _, per = timed_ops([("dx_fp8", lambda: rd.ragged_dot_fp8(dy8, w8, gs3, trans_rhs=True, out=dx))], steps, 3)
    dw8 = torch.empty((64, k, n), dtype=torch.bfloat16, device="cuda")
    _, _, per2 = timed_ops([("dw_fp8", lambda: rd.trans_ragged_dot_fp8(x8, dy8, gs3, out=dw8))], steps, 3)
    per.update(per2)
    for key in ("dx_fp8", "dw_fp8"):
        out[f"backward_m32768_{key}"] = {"ms": round(per[key], 4), "TFLOP/s": round(fl / per[key] / 1e9, 1),
                                        "mfma_frac_fp8": round(fl / per[key] / 1e9 / MFMA_FP8_PEAK_TFLOPS, 4)}
    shares8 = {}
    for pct, hot_rows in (("60", 19660),) + HOT_SHARES:
        gsx = torch.tensor(workloads.hot_expert_sizes(hot_rows=hot_rows), dtype=torch.int32, device="cuda")
        _, _, per_x = timed_ops([
            ("split", lambda: rd.trans_ragged_dot_fp8(x8, dy8, gsx, out=dw8)),
            ("unsplit", lambda: rd.trans_ragged_dot_fp8(x8, dy8, gsx, out=dw8, row_split=False)),
        ], steps, 3)
        shares8[pct] = {key: round(ms, 4) for key, ms in per_x.items()}
    hot_shares["fp8"] = shares8
    out["backward_m32768_hot_expert_dw_by_share"] = hot_shares
    del dy8, w8, x8, dx, dw8
    torch.cuda.empty_cache()
    d = workloads.make(4, "cuda", parts=("x", "w", "fused", "d_out"))
    off = torch.tensor([96], dtype=torch.int32, device="cuda")
    lim = torch.tensor([d["limit"]], dtype=torch.int32, device="cuda")
    o = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device="cuda")
    gb = torch.empty((d["m"], 2 * d["n"]), dtype=torch.bfloat16, device="cuda")
    _, _, per = timed_ops([
        ("window_ragged_dot", lambda: rd.ragged_dot(d["x"], d["w"], d["gs"], off, lim, out=o)),
        ("glu_fwd", lambda: rd.glu_fwd(d["fused"], lim, out=g)),
        ("glu_bwd", lambda: rd.glu_bwd(d["fused"], d["d_out"], lim, out=gb)),
    ], steps, 3)
    L, h = d["limit"], d["n"]
    gsz = d["gs_host"].astype("int64")
    lo, hi = int(gsz[:96].sum()), int(gsz[:128].sum())
    win_rows = hi - lo
    fl = 2.0 * win_rows * d["k"] * d["n"]
    nb = win_rows * d["k"] * 2 + d["w"].numel() * 2 + L * d["n"] * 2
    ms = per["window_ragged_dot"]
    tr = measured_traffic(PACKED_TRAFFIC_FILE)
    out["window_limit_ragged_dot"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                      "GB/s": round(nb / ms / 1e6, 1), "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4),
                                      "algorithmic_bytes": int(nb),
                                      "traffic": None if "ragged_dot" not in tr else int(tr["ragged_dot"])}
    # the same forward with the heaviest ranks of Zipf(1.1) sizes inside the window (a hot window)
    hs = workloads.hot_window_sizes()
    gsh = torch.tensor(hs, dtype=torch.int32, device="cuda")
    _, _, per_h = timed_ops([("hot", lambda: rd.ragged_dot(d["x"], d["w"], gsh, off, lim, out=o))], steps, 3)
    hrows = int(hs[96:128].astype("int64").sum())
    flh = 2.0 * hrows * d["k"] * d["n"]
    out["window_limit_ragged_dot_hot_window"] = {
        "ms": round(per_h["hot"], 4), "TFLOP/s": round(flh / per_h["hot"] / 1e9, 1),
        "mfma_frac": round(flh / per_h["hot"] / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4), "window_rows": hrows,
        "sizes": "Zipf(1.1) over 256 groups, the 32 heaviest ranks in the window 96..127"}
    for key, nbytes in (("glu_fwd", L * h * 6), ("glu_bwd", L * h * 10)):
        out[f"window_limit_{key}"] = {"ms": round(per[key], 4), "GB/s": round(nbytes / per[key] / 1e6, 1),
                                      "hbm_frac": round(nbytes / per[key] / 1e6 / HBM_PEAK_GBS, 4),
                                      "algorithmic_bytes": int(nbytes),
                                      "traffic": None if key not in tr else int(tr[key])}
    del d, o, g, gb
    torch.cuda.empty_cache()
    # weighted unsort backward over the packed buffer's valid rows
    d = workloads.make(4, "cuda", parts=("ug", "uy", "uw"))
    hid = d["k"]
    grad = torch.empty((d["m"], hid), dtype=torch.bfloat16, device="cuda")
    dot = torch.empty((d["m"],), dtype=torch.float32, device="cuda")
    _, _, per = timed_ops([("unsort", lambda: rd.unsort_bwd_rows(d["ug"], d["uy"], d["uw"], lim, grad=grad, dot=dot))],
                          steps, 3)
    nbytes = L * (3 * hid * 2 + 8)  # g, y read, grad written (bf16); w read, dot written (f32)
    out["window_limit_unsort_bwd_rows"] = {"ms": round(per["unsort"], 4), "GB/s": round(nbytes / per["unsort"] / 1e6, 1),
                                           "hbm_frac": round(nbytes / per["unsort"] / 1e6 / HBM_PEAK_GBS, 4),
                                           "algorithmic_bytes": int(nbytes),
                                           "traffic": None if "unsort_bwd_rows" not in tr else int(tr["unsort_bwd_rows"])}
    del d, grad, dot
    torch.cuda.empty_cache()
    out.update(mlp_layer(steps))
    return out


def glu_epilogue(steps):
    """The up-projection forward (m8192 k4096 h1024 g64) with the GLU as the GEMM's epilogue, writing act
    alone or act and the [gate | up] buffer, against ragged_dot followed by glu_fwd."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    d = workloads.make(2, "cuda", parts=("x", "w"))
    x, w, gs = d["x"], d["w"], d["gs"]
    m, k, n = d["m"], d["k"], d["n"]
    rows = int(d["gs_host"].sum())
    fused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((m, n // 2), dtype=torch.bfloat16, device="cuda")

    def separate():
        rd.ragged_dot(x, w, gs, out=fused)
        rd.glu_fwd(fused, out=act)

    _, _, per = timed_ops([
        ("separate", separate),
        ("fused_act_only", lambda: rd.ragged_dot_glu(x, w, gs, act=act)),
        ("fused_act_and_buffer", lambda: rd.ragged_dot_glu(x, w, gs, act=act, fused=fused)),
    ], steps, 3)
    fl = 2.0 * rows * k * n
    out = {f"upproj_fwd_glu_{key}": {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1)}
           for key, ms in per.items()}
    # the same forward with fp8 (E4M3) operands, plain form: half the weight bytes
    x8, w8 = x.to(torch.float8_e4m3fn), w.to(torch.float8_e4m3fn)
    o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    _, _, per = timed_ops([("fp8", lambda: rd.ragged_dot_fp8(x8, w8, gs, out=o))], steps, 3)
    ms = per["fp8"]
    nb = rows * k + w8.numel() + rows * n * 2
    out["upproj_fwd_fp8"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                             "GB/s": round(nb / ms / 1e6, 1), "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)}
    return out


def mlp_layer(steps):
    """The whole MoE expert MLP through the autograd wrapper, forward and backward: wi [64, 4096, 2048]
    as [gate | up], GLU, wo [64, 1024, 4096], on the up-projection's 8192 rows and Zipf(1.1) sizes."""
    import torch

    from expert_ffn_ragged_amd import autograd as ag
    from expert_ffn_ragged_amd import workloads

    d = workloads.make(2, "cuda", parts=("x", "w"))
    x = d["x"].requires_grad_(True)
    wi = d["w"].requires_grad_(True)
    wo = workloads.bf16_normal((64, 1024, 4096), 0.02, 2007, "cuda").requires_grad_(True)
    dout = workloads.bf16_normal((d["m"], 4096), 1.0, 2008, "cuda")
    rows = int(d["gs_host"].sum())

    def step():
        out = ag.moe_mlp(x, wi, wo, d["gs"])
        torch.autograd.grad(out, (x, wi, wo), dout)

    _, _, per = timed_ops([("mlp", step)], steps, 3)
    flop = 3 * (2.0 * rows * 4096 * 2048 + 2.0 * rows * 1024 * 4096)
    return {"moe_mlp_fwd_bwd_m8192_d4096_h1024_g64": {"ms": round(per["mlp"], 4),
                                                     "TFLOP/s": round(flop / per["mlp"] / 1e9, 1),
                                                     "mfma_frac": round(flop / per["mlp"] / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}}


def api_region(iters=5):
    """A region for a HIP API trace (rocprofv3 --hip-trace --memory-copy-trace): the decode layer
    (ragged_dot -> GLU, eagerly and as a replayed graph, group_sizes rewritten on the device between
    replays) and the up-projection step, ``iters`` times, between two hipMemGetInfo calls that mark it.
    Everything is allocated and captured before the first mark; inside the region only the library's
    calls and device-side copies run, so any copy to the host, synchronization or allocation the
    trace shows there would be the library's."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    d5 = workloads.make(5, "cuda", parts=("x", "w"))
    x5, w5, gs5 = d5["x"], d5["w"], d5["gs"]
    m5, n5 = d5["m"], d5["n"]
    gs_alt = torch.roll(gs5, 1)
    gs_now = gs5.clone()
    ws = torch.empty(max(rd.library().rd_forward_workspace_size(m5, d5["k"], n5, d5["G"], 0), 16),
                     dtype=torch.uint8, device="cuda")
    o5 = torch.empty((m5, n5), dtype=torch.bfloat16, device="cuda")
    a5 = torch.empty((m5, n5 // 2), dtype=torch.bfloat16, device="cuda")

    def decode_layer():
        rd.ragged_dot(x5, w5, gs_now, out=o5, workspace=ws)
        rd.glu_fwd(o5, out=a5)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_layer()
    d = workloads.make(2, "cuda", parts=("x", "w"))
    x, w, gs = d["x"], d["w"], d["gs"]
    m, k, n = d["m"], d["k"], d["n"]
    d_act = workloads.bf16_normal((m, n // 2), 1.0, 2006, "cuda")
    fused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((m, n // 2), dtype=torch.bfloat16, device="cuda")
    dfused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((w.shape[0], k, n), dtype=torch.bfloat16, device="cuda")
    wst = torch.empty(max(rd.trans_workspace_size(m, k, n, w.shape[0]), 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.mem_get_info()  # region start mark
    for i in range(iters):
        decode_layer()
        gs_now.copy_(gs_alt if i % 2 == 0 else gs5)  # device-to-device rewrite of group_sizes
        graph.replay()
        rd.ragged_dot(x, w, gs, out=fused)
        rd.glu_fwd(fused, out=act)
        rd.glu_bwd(fused, d_act, out=dfused)
        rd.ragged_dot(dfused, w, gs, trans_rhs=True, out=dx)
        rd.trans_ragged_dot(x, dfused, gs, out=dw, workspace=wst)
    torch.cuda.mem_get_info()  # region end mark
    torch.cuda.synchronize()
    print(json.dumps({"api_region": "done", "iters": iters}), flush=True)


def cpu_info():
    """CPU model (from /proc/cpuinfo), the cores this process may run on, and numpy's BLAS threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    blas = None
    try:
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS defaults to the affinity set
        blas = affinity
    return model, affinity, int(blas)


def cpu_baseline(x, w, dy, gs_host, budget_s=15.0):
    """The CPU oracle, as it stands, on a bounded sample of the headline workload.

    Runs the oracle's trans_rhs ragged_dot (dx) and trans_ragged_dot (dW) expert by expert, largest
    expert first, on the same tensors the GPU just processed (copied to the host one expert at a
    time), until about ``budget_s`` seconds are spent.
    """
    import numpy as np

    import oracle
    from expert_ffn_ragged_amd.workloads import bits

    model, affinity, blas = cpu_info()
    lb = np.concatenate([[0], np.cumsum(gs_host)])
    k, n = w.shape[1], w.shape[2]
    spent, rows, experts = 0.0, 0, 0
    for j in np.argsort(-gs_host, kind="stable"):
        r0, r1 = int(lb[j]), int(lb[j + 1])
        if r1 == r0:
            continue
        xb, dyb, wb = bits(x[r0:r1]), bits(dy[r0:r1]), bits(w[j:j + 1])
        one = np.array([r1 - r0], dtype=np.int32)
        t0 = time.perf_counter()
        oracle.ragged_dot(dyb, wb, one, trans_rhs=True)
        oracle.trans_ragged_dot(xb, dyb, one)
        spent += time.perf_counter() - t0
        rows += r1 - r0
        experts += 1
        if spent >= budget_s:
            break
    flop = 2 * 2.0 * rows * k * n
    nz = int((gs_host > 0).sum())
    # the elementwise GLU oracle (single-threaded NumPy, its exp written out step by step) on 4096 rows of a
    # [gate | up] buffer, h = 1024
    from expert_ffn_ragged_amd.workloads import bf16_normal

    fused = bits(bf16_normal((4096, 2048), 1.0, 4004, "cpu"))
    t0 = time.perf_counter()
    oracle.glu_fwd(fused)
    glu_s = time.perf_counter() - t0
    return {"value": round(flop / spent / 1e12, 6), "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "sample": f"oracle trans_rhs ragged_dot (dx) + trans_ragged_dot (dW), float64, on the timed backward "
                      f"tensors, {experts} of {nz} non-empty experts largest first ({rows} of {int(gs_host.sum())} "
                      f"rows), {spent:.1f} s",
            "cpu_model": model, "affinity_cores": affinity, "blas_threads": blas,
            "glu_fwd": {"value": round(4096 * 6 * 1024 / glu_s / 1e9, 4), "unit": "GB/s", "cores": 1,
                        "sample": f"oracle glu_fwd on 4096 rows, h 1024 (float32 NumPy), {glu_s:.3f} s"}}


def sweep(steps):
    """Every tile shape of every grouped GEMM on the five workloads: one JSON line per (op, tile) with its
    mean time, one summary line per op (the built-in choice and the fastest shape), then the whole table
    as Markdown (ms; "default" is the built-in choice from m, k, n and num_local)."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    cases = []
    d1 = workloads.make(1, "cuda")
    w1t = d1["w"].transpose(1, 2).contiguous()
    o1 = torch.empty((d1["m"], d1["n"]), dtype=torch.bfloat16, device="cuda")
    o1t = torch.empty((d1["m"], d1["k"]), dtype=torch.bfloat16, device="cuda")
    dw1 = torch.empty((4, d1["k"], d1["n"]), dtype=torch.bfloat16, device="cuda")
    cases += [("tiny_ragged_dot", "fwd", lambda: rd.ragged_dot(d1["x"], d1["w"], d1["gs"], out=o1)),
              ("tiny_trans_rhs", "fwd", lambda: rd.ragged_dot(d1["dy"], d1["w"], d1["gs"], trans_rhs=True, out=o1t)),
              ("tiny_trans_ragged_dot", "trans", lambda: rd.trans_ragged_dot(d1["x"], d1["dy"], d1["gs"], out=dw1))]
    del w1t
    d2 = workloads.make(2, "cuda", parts=("x", "w", "dy"))
    m2, k2, n2 = d2["m"], d2["k"], d2["n"]
    o2 = torch.empty((m2, n2), dtype=torch.bfloat16, device="cuda")
    dx2 = torch.empty((m2, k2), dtype=torch.bfloat16, device="cuda")
    dw2 = torch.empty((64, k2, n2), dtype=torch.bfloat16, device="cuda")
    act2 = torch.empty((m2, n2 // 2), dtype=torch.bfloat16, device="cuda")
    cases += [("upproj_ragged_dot", "fwd", lambda: rd.ragged_dot(d2["x"], d2["w"], d2["gs"], out=o2)),
              ("upproj_ragged_dot_glu", "fwd", lambda: rd.ragged_dot_glu(d2["x"], d2["w"], d2["gs"], act=act2)),
              ("upproj_dx_trans_rhs", "fwd",
               lambda: rd.ragged_dot(d2["dy"], d2["w"], d2["gs"], trans_rhs=True, out=dx2)),
              ("upproj_dw_trans_ragged_dot", "trans", lambda: rd.trans_ragged_dot(d2["x"], d2["dy"], d2["gs"],
                                                                                    out=dw2))]
    d3 = workloads.make(3, "cuda")
    dx3 = torch.empty((d3["m"], d3["k"]), dtype=torch.bfloat16, device="cuda")
    dw3 = torch.empty((64, d3["k"], d3["n"]), dtype=torch.bfloat16, device="cuda")
    cases += [("backward_dx_trans_rhs", "fwd",
               lambda: rd.ragged_dot(d3["dy"], d3["w"], d3["gs"], trans_rhs=True, out=dx3)),
              ("backward_dw_trans_ragged_dot", "trans", lambda: rd.trans_ragged_dot(d3["x"], d3["dy"], d3["gs"],
                                                                                      out=dw3))]
    d4 = workloads.make(4, "cuda", parts=("x", "w"))
    off4 = torch.tensor([96], dtype=torch.int32, device="cuda")
    lim4 = torch.tensor([d4["limit"]], dtype=torch.int32, device="cuda")
    o4 = torch.empty((d4["m"], d4["n"]), dtype=torch.bfloat16, device="cuda")
    cases += [("window_limit_ragged_dot", "fwd", lambda: rd.ragged_dot(d4["x"], d4["w"], d4["gs"], off4, lim4,
                                                                       out=o4))]
    d5 = workloads.make(5, "cuda", parts=("x", "w"))
    o5 = torch.empty((d5["m"], d5["n"]), dtype=torch.bfloat16, device="cuda")
    cases += [("decode_ragged_dot_tile_path", "fwd", lambda: rd.ragged_dot(d5["x"], d5["w"], d5["gs"], out=o5))]
    ntile = rd.tile_count()
    with rd.tuning(decode=False):  # warm every case (and the clocks) before timing any
        for _ in range(3):
            for _, _, fn in cases:
                fn()
        torch.cuda.synchronize()
    table = {}
    for name, kind, fn in cases:
        times = {}
        for tile in list(range(ntile)) + [None]:
            kw = {"fwd_tile" if kind == "fwd" else "trans_tile": tile, "decode": False}
            with rd.tuning(**kw):
                _, _, per = timed_ops([(name, fn)], steps, 2)
            times["default" if tile is None else tile] = per[name]
            print(json.dumps({"sweep": name, "tile": "default" if tile is None else tile,
                              "ms": round(per[name], 4)}), flush=True)
        best = min((t for t in times if t != "default"), key=lambda t: times[t])
        print(json.dumps({"sweep_summary": name, "default_ms": round(times["default"], 4), "best_tile": best,
                          "best_ms": round(times[best], 4)}), flush=True)
        table[name] = times
    print("| op | default | " + " | ".join(str(t) for t in range(ntile)) + " |")
    print("|---|---|" + "---|" * ntile)
    for name, times in table.items():
        best = min(times.values())
        cell = lambda v: f"**{v:.3f}**" if v == best else f"{v:.3f}"
        print(f"| {name} | {cell(times['default'])} | " + " | ".join(cell(times[t]) for t in range(ntile)) + " |")
    del d1, d2, d3, d4, d5
    torch.cuda.empty_cache()


def profile_run(which, steps, warmup, cold=False, settle_steps=0):
    """One workload's kernels and nothing else (no timing, no oracle), for rocprofv3 runs; with cold, the
    caches are flushed before every pass as in the headline's timing; settle_steps untimed passes (flushed
    too, with cold) come first, as before the headline's timed loops."""
    import torch

    from expert_ffn_ragged_amd import rd, workloads

    ops = []
    if which == "backward":
        d = workloads.make(3, "cuda")
        dx = torch.empty((d["m"], d["k"]), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((d["G"], d["k"], d["n"]), dtype=torch.bfloat16, device="cuda")
        ops = [lambda: rd.ragged_dot(d["dy"], d["w"], d["gs"], trans_rhs=True, out=dx),
               lambda: rd.trans_ragged_dot(d["x"], d["dy"], d["gs"], out=dw)]
    elif which == "upproj":
        d = workloads.make(2, "cuda", parts=("x", "w"))
        m, k, n = d["m"], d["k"], d["n"]
        x, w, gs = d["x"], d["w"], d["gs"]
        d_act = workloads.bf16_normal((m, n // 2), 1.0, 2006, "cuda")
        fused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        act = torch.empty((m, n // 2), dtype=torch.bfloat16, device="cuda")
        dfused = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((w.shape[0], k, n), dtype=torch.bfloat16, device="cuda")
        ops = [lambda: rd.ragged_dot(x, w, gs, out=fused), lambda: rd.glu_fwd(fused, out=act),
               lambda: rd.glu_bwd(fused, d_act, out=dfused),
               lambda: rd.ragged_dot(dfused, w, gs, trans_rhs=True, out=dx),
               lambda: rd.trans_ragged_dot(x, dfused, gs, out=dw)]
    elif which == "decode":
        d = workloads.make(5, "cuda", parts=("x", "w"))
        o = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(rd.library().rd_forward_workspace_size(d["m"], d["k"], d["n"], d["G"], 0), 16),
                         dtype=torch.uint8, device="cuda")
        ops = [lambda: rd.ragged_dot(d["x"], d["w"], d["gs"], out=o, workspace=ws)]
    else:  # the packed expert buffer at limit 126156: the window+limit forward, GLU fwd / bwd, unsort backward
        d = workloads.make(4, "cuda", parts=("x", "w", "fused", "d_out", "ug", "uy", "uw"))
        lim = torch.tensor([d["limit"]], dtype=torch.int32, device="cuda")
        off = torch.tensor([d["offset"]], dtype=torch.int32, device="cuda")
        o = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device="cuda")
        g = torch.empty((d["m"], d["n"]), dtype=torch.bfloat16, device="cuda")
        gb = torch.empty((d["m"], 2 * d["n"]), dtype=torch.bfloat16, device="cuda")
        grad = torch.empty((d["m"], d["k"]), dtype=torch.bfloat16, device="cuda")
        dot = torch.empty((d["m"],), dtype=torch.float32, device="cuda")
        ops = [lambda: rd.ragged_dot(d["x"], d["w"], d["gs"], off, lim, out=o),
               lambda: rd.glu_fwd(d["fused"], lim, out=g), lambda: rd.glu_bwd(d["fused"], d["d_out"], lim, out=gb),
               lambda: rd.unsort_bwd_rows(d["ug"], d["uy"], d["uw"], lim, grad=grad, dot=dot)]
    if settle_steps:
        settle([(None, fn) for fn in ops], settle_steps, cold)
    for _ in range(warmup + steps):
        if cold:
            flush_caches()
        for fn in ops:
            fn()
    torch.cuda.synchronize()
    print(json.dumps({"profile": which, "launches_per_op": settle_steps + warmup + steps, "settle": settle_steps,
                      "cold": cold}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the ragged-dot kernels run on one MI355X's share of the work; "
              "multi-GPU (expert-parallel) runs are not supported by this benchmark", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from expert_ffn_ragged_amd import rd

    rd.library()
    if args.api_region:
        api_region()
        return
    if args.sweep:
        sweep(max(args.steps, 5))
        return
    if args.profile:
        if args.copy_calib:
            a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            torch.cuda.synchronize()
            del a, b
        profile_run(args.profile, args.steps, args.warmup, args.cold, args.settle)
        return
    if args.copy_calib:
        a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    r = backward(args.steps, args.warmup)
    traffic = measured_traffic(BACKWARD_TRAFFIC_FILE)
    ms_step = r["cold_ms"]
    value = r["step_flop"] / (ms_step * 1e-3) / 1e12
    dom = max(r["cold_per"], key=r["cold_per"].get)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": BACKWARD_WORKLOAD, "m": r["m"], "k": r["k"], "n": r["n"], "groups": r["G"],
                   "valid_rows": r["rows"], "parallelism": "none (1 GPU)"},
        "pct_bf16_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": roofline(dom, r["cold_per"][dom], r["bytes"][dom], r["flops"][dom], traffic.get(dom)),
        "per_kernel": {name: dict(roofline(name, ms, r["bytes"][name], r["flops"][name], traffic.get(name)),
                                  p10_p50_p90_ms=r["cold_pct"][name])
                       for name, ms in r["cold_per"].items()},
        "timing": ("cold: L2 and MALL flushed (512 MiB write) before each step, outside the events; HIP events "
                   "before dx, between dx and dW and after dW on the stream both run on; first "
                   f"{r['settle_steps']} untimed cold steps to reach the steady state of repeated steps, then "
                   "the warmup steps"),
        "warm": {"ms_per_step": round(r["warm_step"], 4),
                 "TFLOP/s": round(r["step_flop"] / r["warm_step"] / 1e9, 1),
                 "per_kernel_ms": {name: round(ms, 4) for name, ms in r["warm_per"].items()},
                 "timing": "steps back to back with events only at the ends; per-kernel times from a separate "
                           "loop with events around each launch"},
    }
    backward_tensors = r["tensors"]
    if not args.headline_only:
        line["extra"] = extra_workloads(max(args.steps, 10), args.warmup)
        if args.all:
            line["extra"].update(extra_all(max(args.steps, 10)))
    line["cpu_baseline"] = None if (args.no_cpu_baseline or args.headline_only) else cpu_baseline(*backward_tensors)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

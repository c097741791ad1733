"""Benchmark of the BFP4/BFP8 weight-streaming matmul path on one MI355X.

Headline step: one decode pass of the dense BFP4 MLP at 27B-class shapes. x is M x 5120
bf16; gate and up (5120 -> 17408, BFP4) run as one streamed GEMV with a fused SwiGLU
epilogue (h kept in fp32), then the BFP4 down projection (17408 -> 5120) writes bf16 y.

The same run also measures the other workloads of the path (one entry each under
"workloads"): the single BFP8 GEMV 2048 x 2048, the dense MLP at M = 8 / 16 / 32, the BFP8
fused QKV / output projections and the 151,936-row LM head at M = 1 and 16, the 256-expert
top-8 BFP4 MoE layer at decode (M = 1 / 8 / 16) and the 2,048-token MoE prefill chunk.

Protocol: inputs are seeded synthetic tensors (the `synth` module), quantized on the GPU
before timing. Packed weights are replicated (or several layers are built) so consecutive
calls read different copies, >= 1 GiB apart in total (more than four times the 256 MB
last-level cache): the bandwidths are HBM numbers. Each timed loop runs W warm-up calls, then
K calls between two events on the launch stream. The headline step is timed as a decode loop
launches it: the K steps (consecutive steps read the weight replicas in turn) captured as one
HIP graph, checked bit for bit against eager steps and replayed once after the W warm-up steps
(another graph's replay). Before the headline's measurements the step runs back to back,
untimed, for --clock-ramp-ms, so that the GPU clocks have left their idle levels, as in a
decode loop that runs without pause; the same graph measurement taken before that ramp, and
the eager time, are reported beside it. Bandwidth = algorithmic bytes (packed
weights actually read + activations in + outputs out) / time per call. The dominant kernel
of the headline step (gate/up + SwiGLU GEMV) is timed alone over K back-to-back launches for
the roofline entry. The CPU oracle is timed on the host: the headline step whole, and one
call (or a bounded sample) of each other workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--M 1] [--quick]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "achieved HBM GB/s (% of peak) + µs/call, BFP4/BFP8 GEMV & MoE at M=1..32"
HIDDEN, INTER = 5120, 17408
MIN_ROTATION = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--clock-ramp-ms", type=float, default=300.0,
                    help="untimed: run the headline step back to back for this long before its "
                         "measurements, so that the GPU clocks are at their working level (0: off)")
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--quick", action="store_true", help="headline step only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-driver", action="store_true",
                    help="only launch the headline gate/up kernel and a 512 MiB copy (run under rocprofv3 --pmc)")
    ap.add_argument("--pmc-report", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of --pmc-driver "
                         "into the traffic summary")
    ap.add_argument("--attn-driver", action="store_true",
                    help="only time the decode-attention workloads and print their lines (run under rocprofv3)")
    ap.add_argument("--moe-driver", action="store_true",
                    help="only time the MoE workloads (decode and the 2,048-token prefill) and print their lines")
    ap.add_argument("--kernel-summary", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace output folder into a per-kernel markdown table")
    ap.add_argument("--counter-driver", action="store_true",
                    help="only launch the decode workloads (16 calls each over cold replicas, between marker "
                         "kernels) and a 512 MiB copy, for rocprofv3 --pmc passes")
    ap.add_argument("--counter-report", nargs="+", metavar="PMC_DIR",
                    help="turn rocprofv3 --pmc folders of --counter-driver (any counters among FETCH_SIZE, "
                         "WRITE_SIZE, TCC_HIT_sum, TCC_MISS_sum, SQ_INSTS_VALU, GRBM_GUI_ACTIVE) into a "
                         "per-workload, per-kernel table")
    ap.add_argument("--floor-driver", action="store_true",
                    help="only time the launch floor: a one-element fill kernel, eager and graph-replayed")
    ap.add_argument("--busy-segments", action="store_true",
                    help="after timing each workload, run 20 more calls between two marker kernels "
                         "(for a per-workload device-busy table from a kernel trace)")
    ap.add_argument("--segments", metavar="BENCH_STDERR",
                    help="with --kernel-summary: the stderr of a --busy-segments run; print the "
                         "device-busy time per call of each workload")
    return ap.parse_args()


# ---- HBM traffic of the headline kernel (rocprofv3 counters) ------------------------------

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_bfp4_gateup_m1_hbm_traffic.md")
# the headline kernel's translation unit and every header it includes
HEADLINE_SOURCES = tuple(f"block_float_quantized_amd/csrc/{f}" for f in (
    "gemv_b4_bf16x.hip", "gemv_row.hpp", "gemv_impl.hpp", "bfp_device.hpp", "bfp_internal.hpp", "argmax.hpp"))
HEADLINE_KERNEL = "row_gemv_kernel<4, 2, true, 5, false, 1>"
DOWN_KERNEL = "row_gemv_kernel<4, 1, false, 1, false, 4>"     # the step's down projection
COPY_BYTES = 512 << 20


def headline_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in HEADLINE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter summary, or None
    when there is none or the kernel's sources changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in text.splitlines() if l.startswith(("traffic_bytes_per_launch:",
                                                                              "kernel_sources_sha256:")))
    if fields.get("kernel_sources_sha256", "").strip() != headline_sources_sha256():
        return None
    return int(fields["traffic_bytes_per_launch"].strip())


def pmc_driver():
    """Launch the headline gate/up kernel and the step's down projection over cold replicas, and
    a plain copy of known size."""
    import torch
    import block_float_quantized_amd as bfq
    torch.cuda.set_device(0)
    c, mats = make_mlp(8)
    x = bf16_dev(c["x"])
    h = torch.empty((1, INTER), dtype=torch.float32, device="cuda")
    y = torch.empty((1, HIDDEN), dtype=torch.bfloat16, device="cuda")
    for i in range(24):
        g, u, d = mats[i % len(mats)]
        bfq.bfp_gemm(g, x, w_up=u, out=h)
        bfq.bfp_gemm(d, h, out_dtype=torch.bfloat16, out=y)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log("pmc driver done")


def pmc_report(fetch_dir: str, write_dir: str):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the headline kernel and of the copy;
    the copy (COPY_BYTES read and written) calibrates each counter to bytes."""
    import glob
    import sqlite3

    def averages(d, counter):
        db = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)[0]
        rows = sqlite3.connect(db).execute(
            "select kernel_name, counter_name, value from counters_collection").fetchall()
        acc = {}
        for name, cn, v in rows:
            if cn != counter:
                continue
            key = ("headline" if HEADLINE_KERNEL in name else "down" if DOWN_KERNEL in name
                   else "copy" if "MulFunctor" in name else None)
            if key:
                acc.setdefault(key, []).append(v)
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    f, fn = averages(fetch_dir, "FETCH_SIZE")
    w, wn = averages(write_dir, "WRITE_SIZE")
    kib = COPY_BYTES / 1024
    ff, fw = kib / f["copy"], kib / w["copy"]
    fetch_b = f["headline"] * 1024 * ff
    write_b = w["headline"] * 1024 * fw
    import block_float_quantized_amd as bfq
    alg = 2 * (bfq.exp_bytes(INTER, HIDDEN) + bfq.code_bytes(4, INTER, HIDDEN)) + HIDDEN * 2 + INTER * 4
    print(f"headline kernel: {HEADLINE_KERNEL} ({fn['headline']} dispatches), copy: {fn['copy']} dispatches")
    print(f"FETCH_SIZE KiB/dispatch: headline {f['headline']:.1f}, copy {f['copy']:.1f} "
          f"(copy reads {kib:.0f} KiB: factor {ff:.4f})")
    print(f"WRITE_SIZE KiB/dispatch: headline {w['headline']:.1f}, copy {w['copy']:.1f} "
          f"(copy writes {kib:.0f} KiB: factor {fw:.4f})")
    print(f"scaled HBM bytes per launch: read {fetch_b:.0f}, written {write_b:.0f}; algorithmic {alg}")
    if "down" in f and "down" in w:
        alg_d = bfq.exp_bytes(HIDDEN, INTER) + bfq.code_bytes(4, HIDDEN, INTER) + INTER * 4 + HIDDEN * 2
        print(f"down kernel: {DOWN_KERNEL} ({fn['down']} dispatches): FETCH_SIZE {f['down']:.1f} KiB, "
              f"WRITE_SIZE {w['down']:.1f} KiB per dispatch; scaled read {f['down'] * 1024 * ff:.0f}, "
              f"written {w['down'] * 1024 * fw:.0f}; algorithmic {alg_d}")
    print(f"traffic_bytes_per_launch: {int(round(fetch_b + write_b))}")
    print(f"kernel_sources_sha256: {headline_sources_sha256()}")


def short_kernel_name(name: str) -> str:
    """Kernel name without return type, namespaces and parameter list (template arguments kept)."""
    import re
    n = name[5:] if name.startswith("void ") else name
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):           # drop the parameter list: the last '(' at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            cut = i
    n = n[:cut]
    n = re.sub(r"\(anonymous namespace\)::", "", n)
    n = re.sub(r"\b(bfp|at::native|std|gemv_detail|mg|am)::", "", n)
    if len(n) > 100:                     # library kernels with lambda-laden template arguments
        n = n[:n.index("<")] + "<...>" if "<" in n else n[:100] + "..."
    return n


def kernel_summary(trace_dir: str):
    """Per-kernel call count, average / min / max duration and share of kernel time."""
    import glob
    import sqlite3
    db = glob.glob(os.path.join(trace_dir, "**", "*.db"), recursive=True)[0]
    rows = sqlite3.connect(db).execute("select name, start, end from kernels").fetchall()
    acc = {}
    for name, t0, t1 in rows:
        acc.setdefault(short_kernel_name(name), []).append((t1 - t0) / 1000.0)
    total = sum(sum(v) for v in acc.values())
    print("| kernel | calls | avg (us) | min (us) | max (us) | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for k, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
              f"{100 * sum(v) / total:.1f}% |")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


BUSY = {"on": False}
BUSY_CALLS = 20
MARKER_KERNEL = "spin_kernel"      # torch.cuda._sleep
MARKER_MAX_NS = 20_000             # a marker spin (1000 cycles) lasts a few us; the spin ahead of
                                   # a timed graph replay (GRAPH_LEAD_SPIN) ~85 us, not a marker


def is_marker(name: str, duration_ns) -> bool:
    return MARKER_KERNEL in name and duration_ns < MARKER_MAX_NS


def busy_segment(name: str, fn):
    """BUSY_CALLS calls of fn between two marker kernels (only with --busy-segments): the kernel
    trace then shows exactly this workload's kernels between the markers."""
    if not BUSY["on"]:
        return
    import torch
    torch.cuda.synchronize()
    torch.cuda._sleep(1000)
    for i in range(BUSY_CALLS):
        fn(i)
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    log(f"busy segment: {name}")


def segment_summary(trace_dir: str, stderr_file: str):
    """Device-busy time per call of each workload: the kernels between each pair of marker
    kernels (in launch order), summed and divided by the calls; also the span from the first
    kernel's start to the last one's end per call (busy time plus the gaps between kernels)."""
    import glob
    import sqlite3
    names = [l.split("busy segment: ", 1)[1].strip() for l in open(stderr_file) if "busy segment: " in l]
    db = glob.glob(os.path.join(trace_dir, "**", "*.db"), recursive=True)[0]
    rows = sorted(sqlite3.connect(db).execute("select name, start, end from kernels").fetchall(),
                  key=lambda r: r[1])
    marks = [i for i, r in enumerate(rows) if is_marker(r[0], r[2] - r[1])]
    print(f"| workload | calls | device busy per call (us) | span per call (us) | kernels per call | largest kernel (share) |")
    print("|---|---:|---:|---:|---:|---|")
    for j, name in enumerate(names):
        if 2 * j + 1 >= len(marks):
            break
        seg = rows[marks[2 * j] + 1:marks[2 * j + 1]]
        if not seg:
            continue
        busy = sum(e - b for _, b, e in seg) / 1000.0
        span = (max(e for _, _, e in seg) - min(b for _, b, _ in seg)) / 1000.0
        per = {}
        for n, b, e in seg:
            k = short_kernel_name(n)
            per[k] = per.get(k, 0.0) + (e - b) / 1000.0
        top = max(per.items(), key=lambda kv: kv[1])
        print(f"| {name} | {BUSY_CALLS} | {busy / BUSY_CALLS:.2f} | {span / BUSY_CALLS:.2f} | "
              f"{len(seg) / BUSY_CALLS:.1f} | `{top[0]}` ({100 * top[1] / busy:.0f}%) |")


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def replicas_for(nbytes: int, cap: int = 512) -> int:
    return int(min(cap, max(2, -(-MIN_ROTATION // max(nbytes, 1)))))


def clone(m):
    import block_float_quantized_amd as bfq
    return bfq.BfpMatrix(m.fmt, m.n, m.k, m.exp.clone(), m.code.clone())


def quantize(fmt, w):
    import torch
    import block_float_quantized_amd as bfq
    t = torch.from_numpy(w).to("cuda")
    m = bfq.bfp_quantize(fmt, t)
    del t
    return m


def workspace(nbytes: int):
    import torch
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device="cuda")


def timed(fn, steps, warmup):
    """Average ms per call of fn(i) over `steps` calls after `warmup` calls."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def timed_graph(fn, outs, calls: int = 64, reps: int = 10):
    """Device time per call of short, launch-bound calls: `calls` calls of fn(i) captured once
    into a HIP graph (torch.cuda.CUDAGraph) and replayed `reps` times, so that host overhead
    between launches drops out. First, three replays, each after eager work (the outputs
    zeroed) and a synchronisation, must leave every output tensor in `outs` bit-identical to
    an eager run of the same calls; else (or if capture fails) None."""
    import torch
    try:
        torch.cuda.synchronize()
        for i in range(calls):
            fn(i)
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                fn(i)
        for _ in range(3):
            for o in outs:
                o.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for o, r in zip(outs, ref):
                if not torch.equal(o.view(torch.uint8), r.view(torch.uint8)):
                    log("graph replay differs from the eager calls; graph timing skipped")
                    return None
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        t0.record(stream)
        for _ in range(reps):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / (reps * calls)
        del g
        return ms
    except RuntimeError as e:
        log(f"graph timing skipped: {e}")
        return None


GRAPH_LEAD_SPIN = 200_000   # device clock cycles (torch.cuda._sleep) ahead of a timed graph replay


def graph_steps(fn, outs, steps: int, warmup: int):
    """ms per step over exactly `steps` consecutive steps fn(0), ..., fn(steps - 1) launched as one
    HIP graph replay, after `warmup` steps fn(0), ..., fn(warmup - 1) launched as the replay of a
    second graph (untimed), a synchronisation and a short device spin (so that the start event
    is taken when the device reaches the graph, not while the host still submits it). First,
    three replays of the timed graph (each after eager work that
    zeroes the outputs, and a synchronisation) must leave every tensor in `outs` bit-identical
    to an eager run of the same steps; else (or if capture fails) None. Returns ms per step."""
    import torch
    try:
        torch.cuda.synchronize()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    fn(i)
            return g

        gk = capture(steps)
        gw = capture(warmup) if warmup > 0 else None
        for _ in range(3):
            for o in outs:
                o.zero_()
            torch.cuda.synchronize()
            gk.replay()
            torch.cuda.synchronize()
            for o, r in zip(outs, ref):
                if not torch.equal(o.view(torch.uint8), r.view(torch.uint8)):
                    log("graph replay differs from the eager steps; graph timing skipped")
                    return None
        if gw is not None:
            gw.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        # a device spin ahead of the start event keeps the idle GPU from taking the event at
        # once: the host then finishes submitting the graph's packets while the spin runs,
        # so the timed span holds the K steps and not the host's graph submission
        torch.cuda._sleep(GRAPH_LEAD_SPIN)
        t0.record(stream)
        gk.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        del gk, gw
        return ms
    except RuntimeError as e:
        log(f"graph timing skipped: {e}")
        return None


def clock_ramp(fn, ms: float) -> int:
    """Untimed: calls fn(i) back to back for `ms` milliseconds of wall time (synchronising every
    32 calls), so that the GPU's core and memory clocks leave their idle states before a
    measurement, as in a decode loop that runs without pause. Returns the calls made."""
    import torch
    n, t = 0, time.perf_counter()
    while (time.perf_counter() - t) * 1e3 < ms:
        for _ in range(32):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def add_graph_timing(entry: dict, fn, outs, nbytes: int):
    """Adds the graph-replay time (see timed_graph) and its rate to a workload entry."""
    ms = timed_graph(fn, outs)
    if ms is None:
        entry["us_per_call_graph"] = None
        return
    entry["us_per_call_graph"] = round(ms * 1e3, 2)
    entry["GB/s_graph"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    entry["pct_hbm_peak_graph"] = round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)


# ---- headline: dense BFP4 MLP decode ------------------------------------------------------

def mlp_bytes(m: int) -> dict:
    import block_float_quantized_amd as bfq
    w_gu = bfq.exp_bytes(INTER, HIDDEN) + bfq.code_bytes(4, INTER, HIDDEN)
    w_d = bfq.exp_bytes(HIDDEN, INTER) + bfq.code_bytes(4, HIDDEN, INTER)
    return {
        "gateup_kernel": 2 * w_gu + m * HIDDEN * 2 + m * INTER * 4,   # weights + x in + h out
        "step": 2 * w_gu + w_d + m * HIDDEN * 2 + m * HIDDEN * 2,     # weights + x in + y out
    }


def make_mlp(replicas: int, seed: int = 0):
    import synth
    c = synth.mlp_case(1, seed)
    base = tuple(quantize(4, c[name]) for name in ("wg", "wu", "wd"))
    mats = [base] + [tuple(clone(b) for b in base) for _ in range(replicas - 1)]
    return c, mats


def run_mlp(args, m, mats, xb, batch_invariant=False, graph=False):
    import torch
    import block_float_quantized_amd as bfq
    x = bf16_dev(xb)
    h = torch.empty((m, INTER), dtype=torch.float32, device="cuda")
    y = torch.empty((m, HIDDEN), dtype=torch.bfloat16, device="cuda")
    R = len(mats)
    g0, u0, d0 = mats[0]
    ws_gu = workspace(bfq.bfp_gemm_workspace_bytes(g0, m, u0))
    ws_d = workspace(bfq.bfp_gemm_workspace_bytes(d0, m))

    def step(i):
        g, u, d = mats[i % R]
        bfq.bfp_gemm(g, x, w_up=u, out=h, workspace=ws_gu, batch_invariant=batch_invariant)
        bfq.bfp_gemm(d, h, out_dtype=torch.bfloat16, out=y, workspace=ws_d, batch_invariant=batch_invariant)

    def gateup(i):
        g, u, _ = mats[i % R]
        bfq.bfp_gemm(g, x, w_up=u, out=h, workspace=ws_gu, batch_invariant=batch_invariant)

    cold = None
    if graph and args.clock_ramp_ms > 0:
        # the same measurement without the ramp, for reference
        cold = graph_steps(step, [h, y], args.steps, args.warmup)
        ramp_calls = clock_ramp(step, args.clock_ramp_ms)
    ms_step = timed(step, args.steps, args.warmup)
    ms_gu = timed(gateup, args.steps, args.warmup)
    busy_segment(f"dense BFP4 MLP M={m}" + (" batch-invariant" if batch_invariant else ""), step)
    b = mlp_bytes(m)
    out = {"us_per_call": ms_step * 1e3, "GB/s": b["step"] / (ms_step * 1e-3) / 1e9,
           "gateup_us": ms_gu * 1e3, "gateup_GB/s": b["gateup_kernel"] / (ms_gu * 1e-3) / 1e9,
           "bytes": b["step"], "tok_per_s": m / (ms_step * 1e-3)}
    if graph:
        # the step as a decode loop launches it: from a HIP graph (eager above for reference)
        ms_g = graph_steps(step, [h, y], args.steps, args.warmup)
        if ms_g is not None:
            out.update({"us_per_step_eager": ms_step * 1e3, "us_per_call": ms_g * 1e3,
                        "GB/s": b["step"] / (ms_g * 1e-3) / 1e9, "tok_per_s": m / (ms_g * 1e-3)})
        if cold is not None:
            out.update({"us_per_step_graph_no_ramp": cold * 1e3, "clock_ramp_calls": ramp_calls})
    return out


def cpu_threads() -> int:
    """Host threads the oracle may use: the cores this process may run on, capped by
    OMP_NUM_THREADS when that is set (a shared host may grant only part of its cores)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(env)) if env.isdigit() and int(env) > 0 else n


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class _PackedBank:
    """Expert weights as the oracle's packed bytes (encoded before timing); decoded on every
    call like the GPU streams them."""

    def __init__(self, layer: dict, experts):
        import oracle
        self.fmt, self.hidden, self.inter = 4, layer["hidden"], layer["inter"]
        h, f = self.hidden, self.inter
        self.packed = {}
        for e in experts:
            if e < 0:
                mats = (layer["sh_gate"], layer["sh_up"], layer["sh_down"])
            else:
                mats = (layer["gate"][e * f:(e + 1) * f], layer["up"][e * f:(e + 1) * f],
                        layer["down"][e * h:(e + 1) * h])
            self.packed[e] = [(oracle.encode(w, 4), w.shape) for w in mats]
        self.nbytes = sum(e_.nbytes + c_.nbytes for v in self.packed.values() for (e_, c_), _ in v)

    def expert(self, e: int):
        import oracle
        return tuple(oracle.decode(ex, cc, 4, n, k) for (ex, cc), (n, k) in self.packed[int(e)])


def cpu_baseline(c: dict, xbits: np.ndarray) -> dict:
    """The CPU oracle timed on the host, one call per workload (the LM head and the prefill
    chunk on a bounded sample): decode the packed bytes (encoded before timing, as the GPU's
    weights are quantized before timing) and compute in fp64 with numpy, BLAS threads = the
    host cores this process may use. The headline step is also timed on one thread."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    threads = cpu_threads()
    out = {}

    def mlp_step(packed, x):
        (eg, cg), (n, k) = packed["wg"]
        (eu, cu), _ = packed["wu"]
        h = oracle.swiglu(oracle.gemm(x, oracle.decode(eg, cg, 4, n, k)), oracle.gemm(x, oracle.decode(eu, cu, 4, n, k)))
        (ed, cd), (nd, kd) = packed["wd"]
        return oracle.bf16_round(oracle.gemm(h, oracle.decode(ed, cd, 4, nd, kd)))

    def clock(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # dense MLP step at M = 1 (the headline workload), whole
    packed = {name: (oracle.encode(c[name], 4), c[name].shape) for name in ("wg", "wu", "wd")}
    wbytes = sum(e.nbytes + cc.nbytes for (e, cc), _ in packed.values())
    x = oracle.bf16_to_f64(xbits)
    nbytes = wbytes + xbits.size * 2 * 2
    with threadpool_limits(limits=threads):
        dt = clock(lambda: mlp_step(packed, x))
    with threadpool_limits(limits=1):
        dt1 = clock(lambda: mlp_step(packed, x))
    out["dense BFP4 MLP M=1"] = {"us_per_call": round(dt * 1e6), "GB/s": round(nbytes / dt / 1e9, 4),
                                 "GB/s_1_thread": round(nbytes / dt1 / 1e9, 4), "sample": "whole step"}
    del packed
    log(f"cpu oracle: MLP step {dt:.2f} s ({threads} threads), {dt1:.2f} s (1 thread)")
    with threadpool_limits(limits=threads):
        # single BFP8 GEMV 2048 x 2048, whole
        g = synth.gemv_case(0)
        (e, cc) = oracle.encode(g["w"], 8)
        xg = oracle.bf16_to_f64(g["x"])
        t = clock(lambda: oracle.gemm(xg, oracle.decode(e, cc, 8, 2048, 2048)))
        nb = e.nbytes + cc.nbytes + 2048 * 2 + 2048 * 4
        out["BFP8 GEMV 2048x2048 M=1"] = {"us_per_call": round(t * 1e6), "GB/s": round(nb / t / 1e9, 4),
                                          "sample": "whole call"}
        # LM head at M = 1: the first 16,384 of 151,936 rows
        rows = 16384
        wl = synth.dense_weights(0, 3, "lm", 151936, 2048, 0.02)[:rows]
        (e, cc) = oracle.encode(wl, 8)
        xl = oracle.bf16_to_f64(synth.proj_case(1, 0, with_lm=False)["x"])
        t = clock(lambda: oracle.gemm(xl, oracle.decode(e, cc, 8, rows, 2048)))
        nb = e.nbytes + cc.nbytes + rows * 4
        out["BFP8 LM head 2048->151936 M=1"] = {"us_per_call_full": round(t * 1e6 * 151936 / rows),
                                                "GB/s": round(nb / t / 1e9, 4),
                                                "sample": f"rows 0..{rows} of 151936, time scaled to all rows"}
        del wl
        # MoE decode at M = 1 (router, top-8, 8 experts + shared), whole; and a 256-token
        # sample of the 2,048-token prefill chunk with the skewed router bias
        layer = synth.moe_layer(0)
        xm = synth.moe_tokens(1, 0)
        rt = oracle.route(xm, layer["router"], 8, sh_gate_bits=layer["sh_gate_w"])
        bank = _PackedBank(layer, [-1] + sorted(set(rt["ids"].ravel().tolist())))

        def moe_dec():
            r = oracle.route(xm, layer["router"], 8, sh_gate_bits=layer["sh_gate_w"])
            oracle.moe_decode(bank, xm, r)
        t = clock(moe_dec)
        nb = bank.nbytes + layer["router"].nbytes + layer["sh_gate_w"].nbytes + 2048 * 6
        out["moe decode M=1"] = {"us_per_call": round(t * 1e6), "GB/s": round(nb / t / 1e9, 4), "sample": "whole call"}
        bias = synth.router_bias(0)
        tok = 256
        xp = synth.moe_tokens(2048, 0, cfg_id=5)[:tok]
        rt = oracle.route(xp, layer["router"], 8, bias=bias, sh_gate_bits=layer["sh_gate_w"])
        bank = _PackedBank(layer, [-1] + sorted(set(rt["ids"].ravel().tolist())))

        def moe_pf():
            r = oracle.route(xp, layer["router"], 8, bias=bias, sh_gate_bits=layer["sh_gate_w"])
            oracle.moe_prefill(bank, xp, r)
        t = clock(moe_pf)
        flops = 2.0 * (tok * 8 + tok) * 3 * 2048 * 512
        out["moe prefill M=2048"] = {"tok_per_s": round(tok / t, 1), "TFLOP/s": round(flops / t / 1e12, 5),
                                     "sample": f"tokens 0..{tok} of the 2,048-token chunk ({len(bank.packed) - 1} "
                                               f"experts used), router bias applied"}
        del layer, bank
    head = out["dense BFP4 MLP M=1"]
    return {"value": head["GB/s"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "value_1_thread": head["GB/s_1_thread"],
            "sample": (f"dense BFP4 MLP step at M=1, whole: decode the packed BFP4 bytes (oracle encoding made "
                       f"before timing) + fp64 GEMVs + SwiGLU + bf16 rounding, {wbytes / 1e6:.1f} MB of packed "
                       f"weights in {dt:.2f} s on {threads} BLAS threads ({dt1:.2f} s on 1); per_config has "
                       f"one oracle call per other workload"),
            "per_config": out}


# ---- decode counters ------------------------------------------------------------------------

COUNTER_CALLS = 16


def counter_driver():
    """The decode workloads one after the other, each as COUNTER_CALLS calls over cold weight
    replicas between two marker kernels, then a plain copy of COPY_BYTES (the byte counters'
    calibration). The marker order is the order of `names` (logged)."""
    import torch
    import block_float_quantized_amd as bfq
    import synth
    torch.cuda.set_device(0)

    def segment(name, fn):
        torch.cuda.synchronize()
        torch.cuda._sleep(1000)
        for i in range(COUNTER_CALLS):
            fn(i)
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        log(f"counter segment: {name}")

    c, mats = make_mlp(8)
    x = bf16_dev(c["x"])
    h = torch.empty((1, INTER), dtype=torch.float32, device="cuda")
    y = torch.empty((1, HIDDEN), dtype=torch.bfloat16, device="cuda")
    segment("dense BFP4 MLP M=1", lambda i: (bfq.bfp_gemm(mats[i % 8][0], x, w_up=mats[i % 8][1], out=h),
                                             bfq.bfp_gemm(mats[i % 8][2], h, out_dtype=torch.bfloat16, out=y)))
    for m in (8, 16):
        xm = bf16_dev(synth.mlp_case(m, 0)["x"])
        hm = torch.empty((m, INTER), dtype=torch.float32, device="cuda")
        ymm = torch.empty((m, HIDDEN), dtype=torch.bfloat16, device="cuda")
        g0, u0, d0 = mats[0]
        wsg = workspace(max(bfq.bfp_gemm_workspace_bytes(g0, m, u0), bfq.bfp_gemm_workspace_bytes(d0, m)))
        segment(f"dense BFP4 MLP M={m}",
                lambda i: (bfq.bfp_gemm(mats[i % 8][0], xm, w_up=mats[i % 8][1], out=hm, workspace=wsg),
                           bfq.bfp_gemm(mats[i % 8][2], hm, out_dtype=torch.bfloat16, out=ymm, workspace=wsg)))
    del mats, c
    torch.cuda.empty_cache()
    g = synth.gemv_case(0)
    p1 = synth.proj_case(1, 0, with_lm=False)
    for name, w, xb in (("BFP8 GEMV 2048x2048 M=1", g["w"], g["x"]), ("BFP8 QKV 2048->5120 M=1", p1["wqkv"], p1["x"]),
                        ("BFP8 O 4096->2048 M=1", p1["wo"], p1["xo"]),
                        ("BFP8 LM head 2048->151936 M=1", synth.dense_weights(0, 3, "lm", 151936, 2048, 0.02), p1["x"])):
        base = quantize(8, w)
        R = replicas_for(base.nbytes)
        reps = [base] + [clone(base) for _ in range(R - 1)]
        xx = bf16_dev(xb)
        yy = torch.empty((1, base.n), dtype=torch.float32, device="cuda")
        ws = workspace(bfq.bfp_gemm_workspace_bytes(base, 1))
        segment(name, lambda i: bfq.bfp_gemm(reps[i % R], xx, out=yy, workspace=ws))
        del reps, base
        torch.cuda.empty_cache()
    layer = synth.moe_layer(0)
    q = {k: quantize(4, layer[k]) for k in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")}
    layers = []
    for r in range(4):
        qq = q if r == 0 else {k: clone(v) for k, v in q.items()}
        layers.append(bfq.MoeLayer(256, 8, 2048, 512, bf16_dev(layer["router"]), None, qq["gate"], qq["up"],
                                   qq["down"], qq["sh_gate"], qq["sh_up"], qq["sh_down"], bf16_dev(layer["sh_gate_w"])))
    xs = [bf16_dev(synth.moe_tokens(1, s_)) for s_ in range(8)]
    ym = torch.empty((1, 2048), dtype=torch.float32, device="cuda")
    wsm = torch.empty((bfq.bfp_moe_workspace_bytes(layers[0], 1),), dtype=torch.uint8, device="cuda")
    segment("moe decode M=1", lambda i: bfq.bfp_moe_forward(layers[i % 4], xs[i % 8], out=ym, workspace=wsm))
    del layers, q
    torch.cuda.empty_cache()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log("counter driver done")


def counter_report(dirs):
    """Per workload (segments between marker kernels, in the driver's order) and kernel: the
    mean per dispatch of each counter collected; bytes calibrated by the copy (FETCH_SIZE and
    WRITE_SIZE in KiB), L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS), VALU issue = 4 cycles per
    wave64 VALU instruction per SIMD (1024) over the GPU cycles (GRBM_GUI_ACTIVE / 8 XCDs);
    matrix busy = SQ_VALU_MFMA_BUSY_CYCLES per SIMD over the GPU cycles, LDS active and
    bank-conflict = SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT per CU (256) over the GPU cycles,
    waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES, TA stalled = TA_ADDR_STALLED_BY_TC_CYCLES per CU."""
    import glob
    import sqlite3
    names = ["dense BFP4 MLP M=1", "dense BFP4 MLP M=8", "dense BFP4 MLP M=16", "BFP8 GEMV 2048x2048 M=1",
             "BFP8 QKV 2048->5120 M=1", "BFP8 O 4096->2048 M=1", "BFP8 LM head 2048->151936 M=1", "moe decode M=1"]
    vals = {}        # (segment, kernel) -> counter -> [values]
    dur = {}
    copy = {}
    for d in dirs:
        db = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)[0]
        rows = sqlite3.connect(db).execute(
            "select dispatch_id, kernel_name, counter_name, value, duration from counters_collection "
            "order by dispatch_id").fetchall()
        seg, inside, last = -1, False, None
        for did, kname, cn, v, du in rows:
            if is_marker(kname, du):
                if did != last:
                    inside = not inside
                    if inside:
                        seg += 1
                last = did
                continue
            last = did
            if "MulFunctor" in kname:
                copy.setdefault(cn, []).append(v)
                continue
            if not inside or seg >= len(names):
                continue
            key = (names[seg], short_kernel_name(kname))
            vals.setdefault(key, {}).setdefault(cn, []).append(v)
            dur.setdefault(key, {})[did] = du
    mean = lambda a: sum(a) / len(a)
    kib = COPY_BYTES / 1024
    ff = kib / mean(copy["FETCH_SIZE"]) if "FETCH_SIZE" in copy else None
    fw = kib / mean(copy["WRITE_SIZE"]) if "WRITE_SIZE" in copy else None
    print("| workload | kernel | dispatches | avg (us) | HBM read MB | HBM written MB | L2 hit | VALU issue "
          "| matrix busy | LDS active | LDS bank-conflict | waiting | TA stalled by TC (cycles per CU) |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for (wl, k), cs in vals.items():
        n = len(dur[(wl, k)])
        us = mean(list(dur[(wl, k)].values())) / 1000.0
        rd = f"{mean(cs['FETCH_SIZE']) * 1024 * ff / 1e6:.2f}" if "FETCH_SIZE" in cs and ff else ""
        wr = f"{mean(cs['WRITE_SIZE']) * 1024 * fw / 1e6:.3f}" if "WRITE_SIZE" in cs and fw else ""
        hit = ""
        if "TCC_HIT_sum" in cs and "TCC_MISS_sum" in cs:
            h_, m_ = mean(cs["TCC_HIT_sum"]), mean(cs["TCC_MISS_sum"])
            hit = f"{100 * h_ / max(h_ + m_, 1):.0f}%"
        cyc = mean(cs["GRBM_GUI_ACTIVE"]) / 8 if "GRBM_GUI_ACTIVE" in cs else None
        pct = lambda c_, units: f"{100 * mean(cs[c_]) / units / max(cyc, 1):.0f}%" if c_ in cs and cyc else ""
        valu = f"{100 * mean(cs['SQ_INSTS_VALU']) * 4 / 1024 / max(cyc, 1):.0f}%" if "SQ_INSTS_VALU" in cs and cyc else ""
        mfma, lds, ldc = pct("SQ_VALU_MFMA_BUSY_CYCLES", 1024), pct("SQ_LDS_IDX_ACTIVE", 256), pct("SQ_LDS_BANK_CONFLICT", 256)
        wait = ""
        if "SQ_WAIT_ANY" in cs and "SQ_WAVE_CYCLES" in cs:
            wait = f"{100 * mean(cs['SQ_WAIT_ANY']) / max(mean(cs['SQ_WAVE_CYCLES']), 1):.0f}%"
        ta = f"{mean(cs['TA_ADDR_STALLED_BY_TC_CYCLES']) / 256:,.0f}" if "TA_ADDR_STALLED_BY_TC_CYCLES" in cs else ""
        print(f"| {wl} | `{k}` | {n} | {us:.2f} | {rd} | {wr} | {hit} | {valu} | {mfma} | {lds} | {ldc} | {wait} | {ta} |")
    if ff and fw:
        print(f"\ncalibration: the copy reads and writes {kib:.0f} KiB per dispatch; FETCH_SIZE factor {ff:.4f}, "
              f"WRITE_SIZE factor {fw:.4f}")


# ---- other workloads -----------------------------------------------------------------------

def launch_floor(args):
    """The cost of one dependent kernel launch with no work: a fill of one float, eager and as
    graph-replayed calls (the floor under any short call, one per launch)."""
    import torch
    torch.cuda.set_device(0)
    t = torch.zeros(1, device="cuda")
    fn = lambda i: t.fill_(float(i % 7))
    ms = timed(fn, max(args.steps, 1000), args.warmup)
    g = timed_graph(fn, [t], calls=300, reps=10)
    out = {"launch floor (one-element fill)": {"us_per_call": round(ms * 1e3, 3),
                                               "us_per_call_graph": None if g is None else round(g * 1e3, 3)}}
    log(f"launch floor: {ms * 1e3:.3f} us eager, {out['launch floor (one-element fill)']['us_per_call_graph']} us graph")
    return out


def gemv_workload(args, name, w, fmt, xs_bits, out_dtype="f32", argmax_name=None):
    """Time bfp_gemm on one matrix over cold replicas for each x in xs_bits (dict M -> bits);
    with argmax_name, also bfp_gemm_argmax (greedy pick per row, no outputs written)."""
    import torch
    import block_float_quantized_amd as bfq
    base = quantize(fmt, w)
    R = replicas_for(base.nbytes)
    mats = [base] + [clone(base) for _ in range(R - 1)]
    out = {}
    for m, xb in xs_bits.items():
        x = bf16_dev(xb)
        y = torch.empty((m, base.n), dtype=torch.float32, device="cuda")
        ws = workspace(bfq.bfp_gemm_workspace_bytes(base, m))
        fn = lambda i: bfq.bfp_gemm(mats[i % R], x, out=y, workspace=ws)
        ms = timed(fn, args.steps, args.warmup)
        nbytes = base.nbytes + m * base.k * 2 + m * base.n * 4
        out[f"{name} M={m}"] = {"us_per_call": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                                "bytes": nbytes, "replicas": R, "tok_per_s": round(m / (ms * 1e-3), 1)}
        add_graph_timing(out[f"{name} M={m}"], fn, [y], nbytes)
        busy_segment(f"{name} M={m}", fn)
        log(f"{name} M={m}: {ms * 1e3:.2f} us (graph replay {out[f'{name} M={m}']['us_per_call_graph']} us)")
        if argmax_name:
            idx = torch.empty((m,), dtype=torch.int32, device="cuda")
            val = torch.empty((m,), dtype=torch.float32, device="cuda")
            ws = workspace(bfq.bfp_gemm_argmax_workspace_bytes(base, m))
            fa = lambda i: bfq.bfp_gemm_argmax(mats[i % R], x, idx=idx, val=val, workspace=ws)
            ms = timed(fa, args.steps, args.warmup)
            nbytes = base.nbytes + m * base.k * 2 + m * 8
            out[f"{argmax_name} M={m}"] = {"us_per_call": round(ms * 1e3, 2),
                                           "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                           "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                                           "bytes": nbytes, "replicas": R, "tok_per_s": round(m / (ms * 1e-3), 1)}
            add_graph_timing(out[f"{argmax_name} M={m}"], fa, [idx, val], nbytes)
            busy_segment(f"{argmax_name} M={m}", fa)
            log(f"{argmax_name} M={m}: {ms * 1e3:.2f} us "
                f"(graph replay {out[f'{argmax_name} M={m}']['us_per_call_graph']} us)")
    del mats
    torch.cuda.empty_cache()
    return out


def attn_workloads(args):
    """Decode attention, 35B-class layer (2 KV heads x 256, 16 query heads), one query token
    over L cached tokens: the BFP8 KV cache, and the long-context cache with BFP8 K and 4-bit V
    after a Hadamard rotation; bytes = the cache's K and V codes and exponents."""
    import torch
    import block_float_quantized_amd as bfq
    out = {}
    kvh, hd, hq = 2, 256, 16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    cases = [("BFP8 KV", bfq.KV_V_BFP8, L) for L in (8192, 32768, 131072)]
    cases += [("BFP8-K 4-bit-V (Hadamard)", bfq.KV_V_BFP4_HADAMARD, L) for L in (32768, 131072, 262144)]
    for name, vf, L in cases:
        row = (hd + hd // 16) + ((hd // 2 if vf == bfq.KV_V_BFP4_HADAMARD else hd) + hd // 16)
        per = kvh * L * row
        R = replicas_for(per, cap=16)
        caches = []
        for r in range(R):
            c = bfq.KvCache.empty(kvh, hd, L, v_format=vf)
            k = torch.randn((L, kvh, hd), device="cuda", generator=gen)
            v = torch.randn((L, kvh, hd), device="cuda", generator=gen)
            bfq.bfp_kv_append(c, k, v, 0)
            caches.append(c)
            del k, v
        q = torch.randn((hq, hd), device="cuda", generator=gen)
        y = torch.empty((hq, hd), dtype=torch.float32, device="cuda")
        ws = workspace(bfq.bfp_attn_decode_workspace_bytes(caches[0], hq, L))
        fn = lambda i: bfq.bfp_attn_decode(caches[i % R], q, L, 1.0 / 16, out=y, workspace=ws)
        ms = timed(fn, args.steps, args.warmup)
        key = f"{name} attention decode L={L}"
        out[key] = {"us_per_call": round(ms * 1e3, 2),
                    "GB/s": round(per / (ms * 1e-3) / 1e9, 1),
                    "pct_hbm_peak": round(100 * per / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                    "cache_bytes": per, "replicas": R,
                    "bytes_per_token_layer": kvh * row}
        add_graph_timing(out[key], fn, [y], per)
        busy_segment(key, fn)
        log(f"attention {name} L={L}: {ms * 1e3:.2f} us (graph replay {out[key]['us_per_call_graph']} us)")
        del caches
        torch.cuda.empty_cache()
    return out


def moe_workloads(args):
    import torch
    import block_float_quantized_amd as bfq
    import synth
    out = {}
    layer = synth.moe_layer(0)
    log("MoE layer drawn")
    q = {k: quantize(4, layer[k]) for k in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")}
    expert_bytes = (q["gate"].nbytes + q["up"].nbytes + q["down"].nbytes) // layer["n_experts"]
    shared_bytes = q["sh_gate"].nbytes + q["sh_up"].nbytes + q["sh_down"].nbytes
    router_bytes = layer["router"].nbytes + layer["sh_gate_w"].nbytes
    nl = 4
    layers = []
    for r in range(nl):
        qq = q if r == 0 else {k: clone(v) for k, v in q.items()}
        layers.append(bfq.MoeLayer(256, 8, 2048, 512, bf16_dev(layer["router"]), None, qq["gate"], qq["up"],
                                   qq["down"], qq["sh_gate"], qq["sh_up"], qq["sh_down"],
                                   bf16_dev(layer["sh_gate_w"])))
    del layer
    for m in (1, 8, 16):
        xs = [bf16_dev(synth.moe_tokens(m, s)) for s in range(8)]
        ws = torch.empty((bfq.bfp_moe_workspace_bytes(layers[0], m),), dtype=torch.uint8, device="cuda")
        y = torch.empty((m, 2048), dtype=torch.float32, device="cuda")
        ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
        distinct = []
        for s in range(8):
            bfq.bfp_moe_forward(layers[0], xs[s], out=y, workspace=ws, topk_ids=ids)
            distinct.append(len(np.unique(ids.cpu().numpy())))
        fn = lambda i: bfq.bfp_moe_forward(layers[i % nl], xs[i % 8], out=y, workspace=ws)
        ms = timed(fn, args.steps, args.warmup)
        d = float(np.mean(distinct))
        nbytes = d * expert_bytes + shared_bytes + router_bytes + m * 2048 * 2 + m * 2048 * 4
        out[f"moe decode M={m}"] = {"us_per_call": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                    "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                                    "distinct_experts": d, "bytes": int(nbytes),
                                    "tok_per_s": round(m / (ms * 1e-3), 1)}
        add_graph_timing(out[f"moe decode M={m}"], fn, [y], int(nbytes))
        busy_segment(f"moe decode M={m}", fn)
        log(f"moe decode M={m}: {ms * 1e3:.2f} us, {d:.1f} experts "
            f"(graph replay {out[f'moe decode M={m}']['us_per_call_graph']} us)")
    # prefill chunk: 2,048 tokens with the skewed router bias
    bias = torch.from_numpy(synth.router_bias(0)).to("cuda")
    for L in layers:
        L.router_bias = bias
    m = 2048
    xs = [bf16_dev(synth.moe_tokens(m, s, cfg_id=5)) for s in range(2)]
    ws = torch.empty((bfq.bfp_moe_workspace_bytes(layers[0], m),), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, 2048), dtype=torch.float32, device="cuda")
    ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
    bfq.bfp_moe_forward(layers[0], xs[0], out=y, workspace=ws, topk_ids=ids)
    used = len(np.unique(ids.cpu().numpy()))
    steps = max(10, args.steps // 10)
    ms = timed(lambda i: bfq.bfp_moe_forward(layers[i % nl], xs[i % 2], out=y, workspace=ws), steps, 3)
    busy_segment("moe prefill M=2048", lambda i: bfq.bfp_moe_forward(layers[i % nl], xs[i % 2], out=y, workspace=ws))
    flops = 2.0 * (m * 8 + m) * 3 * 2048 * 512
    router_flops = 2.0 * m * 257 * 2048
    tfs = flops / (ms * 1e-3) / 1e12
    out["moe prefill M=2048"] = {"us_per_call": round(ms * 1e3, 1), "TFLOP/s": round(tfs, 1),
                                 "pct_bf16_mfma_peak": round(100 * tfs / BF16_MFMA_PEAK_TFLOPS, 1),
                                 "expert_GFLOP": round(flops / 1e9, 2), "router_GFLOP": round(router_flops / 1e9, 2),
                                 "experts_used": used, "tok_per_s": round(m / (ms * 1e-3), 1)}
    log(f"moe prefill: {ms * 1e3:.1f} us, {tfs:.1f} TFLOP/s, {used} experts used")
    del layers
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.kernel_summary and args.segments:
        segment_summary(args.kernel_summary, args.segments)
        return
    if args.kernel_summary:
        kernel_summary(args.kernel_summary)
        return
    if args.pmc_report:
        pmc_report(*args.pmc_report)
        return
    if args.counter_report:
        counter_report(args.counter_report)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; run with --gpus 1"}), flush=True)
        sys.exit(2)
    BUSY["on"] = args.busy_segments
    if args.floor_driver:
        print(json.dumps(launch_floor(args)), flush=True)
        return
    if args.pmc_driver:
        pmc_driver()
        return
    if args.counter_driver:
        counter_driver()
        return
    if args.attn_driver:
        print(json.dumps(attn_workloads(args)), flush=True)
        return
    if args.moe_driver:
        print(json.dumps(moe_workloads(args)), flush=True)
        return
    import torch
    import block_float_quantized_amd as bfq
    import synth
    bfq.lib()
    torch.cuda.set_device(0)
    c, mats = make_mlp(8)
    log("MLP weights quantized")
    xb = synth.mlp_case(args.M, 0)["x"] if args.M != 1 else c["x"]
    head = run_mlp(args, args.M, mats, xb, graph=True)
    log(f"MLP M={args.M}: {head['us_per_call']:.2f} us")
    workloads = {f"dense BFP4 MLP M={args.M}": {k: round(v, 2) for k, v in head.items()}}
    if not args.quick:
        for m in (1, 8, 16, 32):
            if m == args.M:
                continue
            r = run_mlp(args, m, mats, synth.mlp_case(m, 0)["x"])
            workloads[f"dense BFP4 MLP M={m}"] = {k: round(v, 2) for k, v in r.items()}
            log(f"MLP M={m}: {r['us_per_call']:.2f} us")
        # one summation order for every M (the matrix-core kernel at M = 1 as well)
        r = run_mlp(args, 1, mats, synth.mlp_case(1, 0)["x"], batch_invariant=True)
        workloads["dense BFP4 MLP M=1 batch-invariant"] = {k: round(v, 2) for k, v in r.items()}
        log(f"MLP M=1 batch-invariant: {r['us_per_call']:.2f} us")
    cpu = None if args.no_cpu_baseline or args.M != 1 else cpu_baseline(c, xb)
    del mats, c
    torch.cuda.empty_cache()
    if not args.quick:
        g = synth.gemv_case(0)
        workloads.update(gemv_workload(args, "BFP8 GEMV 2048x2048", g["w"], 8, {1: g["x"]}))
        p1, p16 = synth.proj_case(1, 0, with_lm=False), synth.proj_case(16, 0, with_lm=False)
        workloads.update(gemv_workload(args, "BFP8 QKV 2048->5120", p1["wqkv"], 8, {1: p1["x"], 16: p16["x"]}))
        workloads.update(gemv_workload(args, "BFP8 O 4096->2048", p1["wo"], 8, {1: p1["xo"], 16: p16["xo"]}))
        del p1, p16
        lm = synth.dense_weights(0, 3, "lm", 151936, 2048, 0.02)
        workloads.update(gemv_workload(args, "BFP8 LM head 2048->151936", lm,
                                       8, {1: synth.proj_case(1, 0, with_lm=False)["x"],
                                           16: synth.proj_case(16, 0, with_lm=False)["x"]},
                                       argmax_name="BFP8 LM head + greedy argmax 2048->151936"))
        del lm
        workloads.update(moe_workloads(args))
        workloads.update(attn_workloads(args))
    line = {
        "metric": METRIC,
        "value": round(head["GB/s"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] * 1e-3, 5),
        "us_per_call": round(head["us_per_call"], 2),
        "us_per_step_eager": round(head["us_per_step_eager"], 2) if "us_per_step_eager" in head else None,
        "us_per_step_graph_no_ramp": round(head["us_per_step_graph_no_ramp"], 2)
                                     if "us_per_step_graph_no_ramp" in head else None,
        "clock_ramp_ms": args.clock_ramp_ms,
        "timing": ("the K steps (weight replicas in turn) as one HIP graph replay, after the W warmup steps "
                   "as another; before both, the step run back to back for clock_ramp_ms (untimed)")
                  if "us_per_step_eager" in head else "eager launches",
        "pct_hbm_peak": round(100 * head["GB/s"] / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"dense BFP4 MLP decode, 27B-class: x {args.M}x5120 bf16, gate/up 5120x17408 "
                               f"BFP4 + SwiGLU (fp32 h), down 17408x5120 BFP4, bf16 out",
                   "M": args.M, "replicas": 8, "bytes_per_step": head["bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(head["gateup_GB/s"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["gateup_GB/s"] / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic() if args.M == 1 else None,
                     "kernel": HEADLINE_KERNEL + " (BFP4 gate+up+SwiGLU, M=1)", "avg_us": round(head["gateup_us"], 2)},
        "workloads": workloads,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the BFP4/BFP8 weight-streaming matmul path on one MI355X.

One step = one decode pass of the dense BFP4 MLP at 27B-class shapes: x is M x 5120 bf16;
gate and up (5120 -> 17408, BFP4) run as one streamed GEMV with a fused SwiGLU epilogue,
then the BFP4 down projection (17408 -> 5120) writes bf16 y. Weights are seeded synthetic
N(0, 0.02) x per-row LogNormal(0, 0.5), quantized on the GPU before timing.

Protocol: the packed weights are replicated so that consecutive steps read different copies
(>= 1 GiB rotation, more than four times the 256 MB last-level cache), so the numbers are
HBM numbers. W warm-up steps, then K timed steps between two events on the launch stream.
The headline value is algorithmic bytes (packed weights + x + y) per step divided by the
step time. The dominant kernel (gate/up + SwiGLU) is also timed launch by launch with events
on the same stream for the roofline entry. The CPU oracle is timed on a bounded sample of
the same work on the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--M 1] [--sweep]
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
METRIC = "achieved HBM GB/s (% of peak) + µs/call, BFP4/BFP8 GEMV & MoE at M=1..32"
HIDDEN, INTER = 5120, 17408


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--sweep", action="store_true", help="also time M = 1, 8, 16, 32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="rows per matrix in the CPU sample")
    return ap.parse_args()


def mlp_bytes(m: int) -> dict:
    import block_float_quantized_amd as bfq
    w_gu = bfq.exp_bytes(INTER, HIDDEN) + bfq.code_bytes(4, INTER, HIDDEN)
    w_d = bfq.exp_bytes(HIDDEN, INTER) + bfq.code_bytes(4, HIDDEN, INTER)
    return {
        "weights": 2 * w_gu + w_d,
        "gateup_kernel": 2 * w_gu + m * HIDDEN * 2 + m * INTER * 4,   # weights + x + h written
        "step": 2 * w_gu + w_d + m * HIDDEN * 2 + m * HIDDEN * 2,     # weights + x in + y out
    }


def run_gpu(args, m: int, mats, x):
    import torch
    import block_float_quantized_amd as bfq
    stream = torch.cuda.current_stream()
    R = len(mats)
    h = torch.empty((m, INTER), dtype=torch.float32, device="cuda")
    y = torch.empty((m, HIDDEN), dtype=torch.bfloat16, device="cuda")

    def step(i, ev=None):
        g, u, d = mats[i % R]
        if ev is not None:
            ev[0].record(stream)
        bfq.bfp_gemm(g, x, w_up=u, out=h, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        bfq.bfp_gemm(d, h, out_dtype=torch.bfloat16, out=y, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # whole-step timing
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # per-launch timing of the dominant kernel (events around each gate/up launch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return ms_step, gu_ms


def make_weights(replicas: int, seed: int = 0):
    import torch
    import block_float_quantized_amd as bfq
    import synth
    c = synth.mlp_case(1, seed)
    base = []
    for name in ("wg", "wu", "wd"):
        w = torch.from_numpy(c[name]).to("cuda")
        base.append(bfq.bfp_quantize(4, w))
        del w
    mats = [tuple(base)]
    for _ in range(replicas - 1):
        mats.append(tuple(bfq.BfpMatrix(b.fmt, b.n, b.k, b.exp.clone(), b.code.clone()) for b in base))
    return c, mats


def cpu_baseline(c: dict, rows: int, xbits: np.ndarray) -> dict:
    """Time the CPU oracle (decode the packed bytes, fp64 GEMV) on `rows` rows of each matrix."""
    import oracle
    from threadpoolctl import threadpool_limits
    m = xbits.shape[0]
    x = oracle.bf16_to_f64(xbits)
    packed = {}
    for name in ("wg", "wu", "wd"):
        w = c[name][:rows]
        packed[name] = (oracle.encode(w, 4), w.shape)
    nbytes = sum(e.nbytes + cc.nbytes for (e, cc), _ in packed.values())
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        (eg, cg), (n, k) = packed["wg"]
        (eu, cu), _ = packed["wu"]
        g = oracle.gemm(x, oracle.decode(eg, cg, 4, n, k))
        u = oracle.gemm(x, oracle.decode(eu, cu, 4, n, k))
        hh = oracle.swiglu(g, u)
        (ed, cd), (nd, kd) = packed["wd"]
        hfull = np.zeros((m, kd))
        hfull[:, :hh.shape[1]] = hh
        oracle.gemm(hfull, oracle.decode(ed, cd, 4, nd, kd))
        dt = time.perf_counter() - t
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} rows of each of gate, up and down (M={m}): decode packed BFP4 + fp64 GEMV, "
                      f"{nbytes / 1e6:.1f} MB of packed weights in {dt:.2f} s, 1 thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
    import torch
    import block_float_quantized_amd as bfq
    bfq.lib()
    torch.cuda.set_device(0)
    import synth
    c, mats = make_weights(args.replicas)
    Ms = [args.M] + ([mm for mm in (1, 8, 16, 32) if mm != args.M] if args.sweep else [])
    results = {}
    for m in Ms:
        xb = synth.mlp_case(m, 0)["x"] if m != 1 else c["x"]
        x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).to("cuda").view(torch.bfloat16)
        ms_step, gu_ms = run_gpu(args, m, mats, x)
        b = mlp_bytes(m)
        results[m] = {
            "ms_per_step": ms_step,
            "gbs": b["step"] / (ms_step * 1e-3) / 1e9,
            "gateup_us": gu_ms * 1e3,
            "gateup_gbs": b["gateup_kernel"] / (gu_ms * 1e-3) / 1e9,
            "step_bytes": b["step"],
        }
    r = results[args.M]
    line = {
        "metric": METRIC,
        "value": round(r["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "us_per_call": round(r["ms_per_step"] * 1e3, 2),
        "pct_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"dense BFP4 MLP decode, 27B-class: x {args.M}x5120 bf16, gate/up 5120x17408 "
                               f"BFP4 + SwiGLU, down 17408x5120 BFP4, bf16 out",
                   "M": args.M, "replicas": args.replicas, "bytes_per_step": r["step_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(r["gateup_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["gateup_gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemv_kernel<BFP4, SwiGLU> (gate+up)", "avg_us": round(r["gateup_us"], 2)},
    }
    if args.sweep:
        line["by_M"] = {str(m): {"us_per_call": round(v["ms_per_step"] * 1e3, 2), "GB/s": round(v["gbs"], 1),
                                 "tok_per_s": round(m / (v["ms_per_step"] * 1e-3), 1)} for m, v in results.items()}
    if not args.no_cpu_baseline:
        xb = synth.mlp_case(args.M, 0)["x"] if args.M != 1 else c["x"]
        line["cpu_baseline"] = cpu_baseline(c, args.cpu_rows, xb)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

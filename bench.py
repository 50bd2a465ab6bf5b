"""Benchmark of the ONNX recurrent-operator hot path on one MI355X.

One step = one full operator invocation (weight pack, state init, the
projection XW = X . W^T over all steps, the step loop with its gate
arithmetic, masking and output writes) on one batch of synthetic input that
is already resident in device memory.  The workload is the bidirectional LSTM
(seq 512, batch 64, input 1024, hidden 1024, fp32, full-length sequences, no
peepholes); its inputs are drawn by workloads.py.

Prints ONE JSON line: throughput in cell-updates/s (seq * batch * dirs per
second), the roofline of the dominant kernel from HIP events recorded on the
library's stream during extra timed runs, and the CPU oracle timed on a
bounded sample of the same workload on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSTM/GRU cell-updates/s (seq·batch·dirs per s) + % of HBM/MFMA roofline, 1 GPU"
FP32_MFMA_PEAK_TFLOPS = 157.3      # MI355X dense fp32 matrix peak
BF16_MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="lstm_bidir_s512_b64_i1024_h1024")
    p.add_argument("--kernel-path", type=int, default=0, help="0 auto, 1 persistent, 2 per step")
    p.add_argument("--cpu-budget-s", type=float, default=30.0, help="0 skips the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def flops_per_run(c):
    """Algorithmic FLOPs of the two products of one invocation (every step of
    every row, i.e. the nominal work; GRU lbr=0's two products per step have
    the same total as one G*H-wide product)."""
    D, G = c.dirs, c.gates
    proj = 2.0 * c.seq * c.batch * D * G * c.hidden * c.input
    rec = 2.0 * c.seq * c.batch * D * G * c.hidden * c.hidden
    return proj, rec


def cpu_baseline(c, budget_s):
    """The oracle (as it is) on a bounded sample of the same workload: every
    batch row, all steps, all directions, run repeatedly until about 10 s (at
    most budget_s) of CPU work has been timed.  Returns cell-updates/s."""
    import oracle
    nt = oracle.default_threads()
    cells = c.seq * c.batch * c.dirs
    t0 = time.perf_counter()
    oracle.run(c, n_threads=nt, want_y=True)
    first = time.perf_counter() - t0
    reps = 1
    if first < 10.0:
        reps = max(1, min(math.ceil(10.0 / max(first, 1e-3)), int(budget_s / max(first, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.run(c, n_threads=nt, want_y=True)
        dt = time.perf_counter() - t0
    else:
        dt = first
    return {"value": cells * reps / dt, "unit": "cell-updates/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole workload ({c.batch} rows x {c.seq} steps x {c.dirs} directions "
                      f"= {cells} cell-updates) run {reps} time(s) in {dt:.1f} s on {nt} threads",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import recurrent_nn_amd as ra
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    ra._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = workloads.workload(args.workload)
    print(f"[bench] workload {c.name}: inputs drawn", file=sys.stderr, flush=True)
    t = {k: (v.to(dev) if v is not None and k != "sequence_lens" else v)
         for k, v in c.tensors().items()}
    plan = ra.plan_for_case(c, kernel_path=args.kernel_path)
    Y = torch.empty(plan.output_shapes()[0], dtype=torch.float32, device=dev)
    Yh = torch.empty(plan.output_shapes()[1], dtype=torch.float32, device=dev)
    Yc = torch.empty_like(Yh) if c.op == "LSTM" else None
    out = (Y, Yh, Yc)
    stream = torch.cuda.current_stream(dev)

    def step():
        plan.run(t["X"], t["W"], t["R"], t["B"], t["sequence_lens"], t["initial_h"],
                 t["initial_c"], t["P"], out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan.check(stream)
    print(f"[bench] {plan.describe()}", file=sys.stderr, flush=True)

    # ---- the timed region: exactly K steps ---------------------------------
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/step (wall {wall:.3f} s)",
          file=sys.stderr, flush=True)

    # ---- per-kernel durations from HIP events on the library's stream -------
    plan.enable_timing(True)
    per = {k: [] for k in ra.STAGES}
    for _ in range(max(3, args.steps)):
        step()
        for k, v in plan.last_timings().items():
            per[k].append(v)
    plan.enable_timing(False)
    torch.cuda.synchronize()
    plan.check(stream)
    stage_ms = {k: float(np.mean(v)) for k, v in per.items()}
    print(f"[bench] stage ms: {json.dumps(stage_ms)}", file=sys.stderr, flush=True)

    proj_f, rec_f = flops_per_run(c)
    proj_peak = BF16_MFMA_PEAK_TFLOPS if c.proj_bf16 else FP32_MFMA_PEAK_TFLOPS
    kernels = {
        "projection": {"bound": "mfma", "flop": proj_f, "ms": stage_ms["projection"],
                       "achieved": proj_f / (stage_ms["projection"] * 1e-3) / 1e12,
                       "peak": proj_peak, "unit": "TFLOP/s"},
        "recurrence": {"bound": "mfma", "flop": rec_f, "ms": stage_ms["recurrence"],
                       "achieved": rec_f / (stage_ms["recurrence"] * 1e-3) / 1e12,
                       "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "us_per_step": stage_ms["recurrence"] * 1e3 / c.seq},
    }
    for k in kernels.values():
        k["frac"] = k["achieved"] / k["peak"]
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    roofline = {"bound": dk["bound"], "achieved": round(dk["achieved"], 3), "peak": dk["peak"],
                "unit": dk["unit"], "frac": round(dk["frac"], 4), "traffic": None,
                "kernel": dom}

    cells = c.cell_updates()
    value = cells / (ms * 1e-3)
    res = {
        "metric": METRIC, "value": value, "unit": "cell-updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+f32" if c.proj_bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": c.name, "op": c.op, "direction": c.direction, "seq": c.seq,
                   "batch": c.batch, "input": c.input, "hidden": c.hidden, "dirs": c.dirs,
                   "layout": c.layout, "global_batch": c.batch, "seq_len": c.seq,
                   "parallelism": "none (1 GPU)", "plan": plan.describe()},
        "valid_cell_updates_per_s": c.valid_cell_updates() / (ms * 1e-3),
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "stage_ms": stage_ms,
    }
    if not args.no_cpu_baseline and args.cpu_budget_s > 0:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(c, args.cpu_budget_s)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

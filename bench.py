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
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSTM/GRU cell-updates/s (seq·batch·dirs per s) + % of HBM/MFMA roofline, 1 GPU"
FP32_MFMA_PEAK_TFLOPS = 157.3      # MI355X dense fp32 matrix peak
BF16_MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
# Exact mode's roof: binary32 multiplies and adds issued separately on the
# vector ALUs.  The published fp32 vector peak (157.3 TFLOP/s = 256 CUs x 4
# SIMDs x 32 lanes x 2 flops x 2.4 GHz) counts a fused multiply-add as two
# flops; with the multiply and the add as two instructions it is half.
FP32_VALU_MULADD_PEAK_TFLOPS = 157.3 / 2
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
    p.add_argument("--exact", action="store_true",
                   help="exact mode: k-ordered unfused products on the VALU (results bit-identical "
                        "to the oracle); reported against the fp32 vector peak")
    p.add_argument("--time-chunk", type=int, default=0, help="steps per time chunk (0: all)")
    p.add_argument("--peaks", action="store_true",
                   help="print library references (HBM copy, fp32/bf16 GEMM) and exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB -> 1 GiB device copy kernel (to scale HBM counters)")
    p.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR"),
                   help="summarise four rocprofv3 --pmc csv runs (FETCH_SIZE / WRITE_SIZE of the "
                        "bench and of --copy-calibration) into per-launch HBM bytes, as JSON")
    p.add_argument("--counter-summary", metavar="PMC_DIR",
                   help="mean of every counter per dispatch of each kernel in a rocprofv3 --pmc "
                        "csv run, as JSON")
    return p.parse_args()


# Source files whose kernels a traffic figure was measured on; a figure whose
# hash no longer matches the tree is stale and not reported.
KERNEL_SOURCES = {
    "recurrence": ["activations.h", "common.h"],     # + every recurrence* file
    "projection": ["proj_gemm.hip", "common.h"],
}
KERNEL_NAMES = {"recurrence": "rec_", "projection": "proj_gemm"}
COPY_BYTES = 1 << 30


def kernel_hash(stage):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_nn_amd", "csrc")
    names = list(KERNEL_SOURCES[stage])
    if stage == "recurrence":
        names += sorted(f for f in os.listdir(csrc) if f.startswith("recurrence"))
    for n in names:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def copy_calibration():
    """A plain elementwise copy (negation) of COPY_BYTES into COPY_BYTES: the
    reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES}), flush=True)


def achievable_peaks():
    """Library references on this part, next to the spec peaks: a plain 1 GiB
    device-to-device copy (HBM read + write), and torch's own fp32 and bf16
    matrix products at the plain shapes of the fp32 (S 512, Bt 64, I 1024,
    G*H*D 8192) and bf16 (S 256, Bt 256, I 2048, G*H 6144) projections, with
    no row gather.  Context only: nothing on the measured path uses them."""
    import torch
    dev = torch.device("cuda:0")

    def ms_per(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = ms_per(lambda: dst.copy_(src), 10)
    del src, dst
    out = {"hbm_copy_gbs": 2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9}
    for name, (M, N, K, dt) in {"fp32_gemm_tflops": (32768, 8192, 1024, torch.float32),
                                "bf16_gemm_tflops": (65536, 6144, 2048, torch.bfloat16)}.items():
        g = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn(M, K, device=dev, generator=g).to(dt)
        b = torch.randn(K, N, device=dev, generator=g).to(dt)      # [K, N], contiguous
        ms = ms_per(lambda: torch.matmul(a, b), 5)
        out[name] = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        del a, b
    out["spec"] = {"hbm_gbs": HBM_PEAK_GBS, "fp32_mfma_tflops": FP32_MFMA_PEAK_TFLOPS,
                   "bf16_mfma_tflops": BF16_MFMA_PEAK_TFLOPS}
    print(json.dumps(out), flush=True)


def _pmc_rows(d, counter=False):
    """(kernel name, dispatch id, [counter name,] counter value) from every
    rocprofv3 counter csv below directory d."""
    import csv
    import glob
    rows = []
    for fn in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                v = float(r["Counter_Value"])
                rows.append((r["Kernel_Name"], int(r["Dispatch_Id"]), r["Counter_Name"], v) if counter
                            else (r["Kernel_Name"], int(r["Dispatch_Id"]), v))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def counter_summary(d):
    """Mean over dispatches of each counter, per kernel (counters of one
    dispatch with several rows, e.g. per dimension, are summed first)."""
    import numpy as np
    acc = {}
    for name, did, ctr, v in _pmc_rows(d, counter=True):
        k = acc.setdefault(name, {}).setdefault(ctr, {})
        k[did] = k.get(did, 0.0) + v
    out = {n: {c: {"mean": float(np.mean(list(v.values()))), "dispatches": len(v)}
               for c, v in cs.items()} for n, cs in acc.items()}
    print(json.dumps(out, indent=1))


def traffic_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, workload):
    """Per-launch HBM bytes of each kernel: mean counter KiB per dispatch,
    scaled by bytes / counter of the plain copy."""
    import numpy as np

    def per_kernel(d):
        acc = {}
        for name, did, v in _pmc_rows(d):
            acc.setdefault(name, {}).setdefault(did, 0.0)
            acc[name][did] += v
        return {k: float(np.mean(list(v.values()))) for k, v in acc.items()}

    def copy_kib(d):
        pk = per_kernel(d)
        name = max(pk, key=pk.get)
        return name, pk[name]

    cname, cf = copy_kib(cfetch_dir)
    _, cw = copy_kib(cwrite_dir)
    rscale, wscale = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    fk, wk = per_kernel(fetch_dir), per_kernel(write_dir)
    out = {"workload": workload, "copy_kernel": cname, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "read_scale": rscale, "write_scale": wscale, "kernels": {}}
    for stage, prefix in KERNEL_NAMES.items():
        names = [n for n in fk if prefix in n]
        if not names:
            continue
        n = max(names, key=fk.get)
        f_kib, w_kib = fk[n], wk.get(n, float("nan"))
        out["kernels"][stage] = {
            "name": n, "fetch_kib": f_kib, "write_kib": w_kib,
            "traffic_bytes": f_kib * 1024.0 * rscale + w_kib * 1024.0 * wscale,
            "source_hash": kernel_hash(stage)}
    print(json.dumps(out, indent=1))


def measured_traffic(workload, stage):
    """Bytes per launch recorded for this kernel and workload, or None when
    absent or taken on different kernel sources."""
    fn = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    try:
        with open(fn) as f:
            k = json.load(f)["kernels"][stage]
    except (OSError, KeyError, ValueError):
        return None
    if k.get("source_hash") != kernel_hash(stage):
        return None
    return k["traffic_bytes"]


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
    dt = first
    if first < 10.0:
        # the first run warms up; then repeat until 10 s are timed, stopping
        # before another run would pass the budget
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.run(c, n_threads=nt, want_y=True)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or dt + dt / reps > budget_s:
                break
    return {"value": cells * reps / dt, "unit": "cell-updates/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole workload ({c.batch} rows x {c.seq} steps x {c.dirs} directions "
                      f"= {cells} cell-updates) run {reps} time(s) in {dt:.1f} s on {nt} threads",
            "seconds": dt}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, workload=args.workload)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the step loop runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import recurrent_nn_amd as ra
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.peaks:
        achievable_peaks()
        return
    ra._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = workloads.workload(args.workload)
    print(f"[bench] workload {c.name}: inputs drawn", file=sys.stderr, flush=True)
    t = {k: (v.to(dev) if v is not None and k != "sequence_lens" else v)
         for k, v in c.tensors().items()}
    plan = ra.plan_for_case(c, kernel_path=args.kernel_path, exact=args.exact,
                            time_chunk=args.time_chunk)
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

    # ---- each invocation timed on its own, for the median and the minimum ----
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in evs:
        a_.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    each = sorted(a_.elapsed_time(b_) for a_, b_ in evs)

    proj_f, rec_f = flops_per_run(c)
    proj_peak = BF16_MFMA_PEAK_TFLOPS if c.proj_bf16 else FP32_MFMA_PEAK_TFLOPS
    bound = "mfma"
    if args.exact:
        proj_peak = rec_peak = FP32_VALU_MULADD_PEAK_TFLOPS
        bound = "alu"
    else:
        rec_peak = FP32_MFMA_PEAK_TFLOPS
    kernels = {
        "projection": {"bound": bound, "flop": proj_f, "ms": stage_ms["projection"],
                       "achieved": proj_f / (stage_ms["projection"] * 1e-3) / 1e12,
                       "peak": proj_peak, "unit": "TFLOP/s"},
        "recurrence": {"bound": bound, "flop": rec_f, "ms": stage_ms["recurrence"],
                       "achieved": rec_f / (stage_ms["recurrence"] * 1e-3) / 1e12,
                       "peak": rec_peak, "unit": "TFLOP/s",
                       "us_per_step": stage_ms["recurrence"] * 1e3 / c.seq},
    }
    for k in kernels.values():
        k["frac"] = k["achieved"] / k["peak"]
    # the recurrence's operand streams per step: R (what a kernel that streamed
    # it would need, against HBM) and the H rows every workgroup reads (L2)
    desc = dict(kv.split("=", 1) for kv in plan.describe().split() if "=" in kv)
    t_step = stage_ms["recurrence"] * 1e-3 / c.seq
    r_bytes = 4.0 * c.dirs * c.gates * c.hidden * c.hidden
    h_bytes = 4.0 * int(desc["workgroups"]) * int(desc["BT"]) * int(desc["Hp"])
    kernels["recurrence"]["r_stream_gbs"] = r_bytes / t_step / 1e9
    kernels["recurrence"]["r_stream_frac_hbm"] = r_bytes / t_step / (HBM_PEAK_GBS * 1e9)
    kernels["recurrence"]["h_broadcast_gbs"] = h_bytes / t_step / 1e9
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    roofline = {"bound": dk["bound"], "achieved": round(dk["achieved"], 3), "peak": dk["peak"],
                "unit": dk["unit"], "frac": round(dk["frac"], 4),
                "traffic": measured_traffic(c.name, dom),
                "kernel": dom}

    cells = c.cell_updates()
    value = cells / (ms * 1e-3)
    res = {
        "metric": METRIC, "value": value, "unit": "cell-updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+f32" if c.proj_bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": c.name, "mode": "exact" if args.exact else "fast",
                   "time_chunk": args.time_chunk, "op": c.op, "direction": c.direction, "seq": c.seq,
                   "batch": c.batch, "input": c.input, "hidden": c.hidden, "dirs": c.dirs,
                   "layout": c.layout, "global_batch": c.batch, "seq_len": c.seq,
                   "parallelism": "none (1 GPU)", "plan": plan.describe()},
        "valid_cell_updates_per_s": c.valid_cell_updates() / (ms * 1e-3),
        "ms_per_step_median": each[len(each) // 2], "ms_per_step_min": each[0],
        "inputs_sha256": c.digests(),
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "stage_ms": stage_ms,
    }
    if not args.no_cpu_baseline and args.cpu_budget_s > 0:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(c, args.cpu_budget_s)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        res["gpu_over_cpu_baseline"] = value / cb["value"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

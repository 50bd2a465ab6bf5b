"""Benchmark of the ONNX recurrent-operator hot path on one MI355X.

One step = one full operator invocation (weight pack, state init, the
projection XW = X . W^T over all steps, the step loop with its gate
arithmetic, masking and output writes) on one batch of synthetic input that
is already resident in device memory.  The headline workload is the
bidirectional LSTM (seq 512, batch 64, input 1024, hidden 1024, fp32,
full-length sequences, no peepholes); its inputs are drawn by workloads.py.

Prints ONE JSON line: throughput in cell-updates/s (seq * batch * dirs per
second) of the headline workload; the roofline of its dominant kernel from
HIP events recorded on the library's stream during extra timed runs, counted
on the valid work (positions past a row's sequence length are not work of the
method); the same figures for the other workloads of the list under
"configs"; and the CPU oracle timed on a bounded sample of the headline
workload on the host's cores.
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
    p.add_argument("--no-configs", action="store_true",
                   help="time only --workload, not the other workloads of the list")
    p.add_argument("--exact", action="store_true",
                   help="exact mode: k-ordered unfused products on the VALU (results bit-identical "
                        "to the oracle); reported against the fp32 vector peak")
    p.add_argument("--time-chunk", type=int, default=0, help="steps per time chunk (0: all)")
    p.add_argument("--fuse-projection", type=int, default=0, choices=(0, 1, 2),
                   help="0 automatic, 1 the projection as its own launch, 2 inside the step loop")
    p.add_argument("--peaks", action="store_true",
                   help="print library references (HBM copy, fp32/bf16 GEMM) and exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB -> 1 GiB device copy kernel (to scale HBM counters)")
    p.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR"),
                   help="summarise four rocprofv3 --pmc csv runs (FETCH_SIZE / WRITE_SIZE of the "
                        "bench and of --copy-calibration) into per-launch HBM bytes, as JSON")
    p.add_argument("--stamps", action="store_true",
                   help="with the instrumented build loaded (RNN_AMD_LIB=recurrent_nn_amd/"
                        "librecurrent_nn_amd_stamps.so, built by `recurrent_nn_amd/build.py "
                        "--stamps`): the step loop's cycle stamps of one workgroup "
                        "(RNN_AMD_STAMP_WG, default 0), median intervals over the steps, as JSON")
    p.add_argument("--counter-summary", metavar="PMC_DIR",
                   help="mean of every counter per dispatch of each kernel in a rocprofv3 --pmc "
                        "csv run, as JSON")
    return p.parse_args()


# Source files whose kernels a traffic figure was measured on; a figure whose
# hash no longer matches the tree is stale and not reported.  The fast step
# loops are defined in the headers below (the four-wave kernel in
# recurrence_kernel.h, the two-half kernel also in recurrence_pipe.h); the
# exact-mode and fused kernels, the launcher and the tables that pick
# instantiations are not part of them.
KERNEL_SOURCES = {
    "recurrence": ["activations.h", "common.h", "recurrence_kernel.h"],
    "projection": ["proj_gemm.hip", "common.h"],
}
KERNEL_EXTRA_SOURCES = {"rec_pipe_kernel": ["recurrence_pipe.h"]}
# the instantiation families a kernel is compiled in (their own device flags
# count too)
KERNEL_FAMILIES = {"rec_kernel": (0, 1, 2), "rec_pipe_kernel": (3,), "rec_fused_kernel": (4,)}
KERNEL_NAMES = {"recurrence": "rec_", "projection": "proj_gemm"}
COPY_BYTES = 1 << 30


def _code_only(text):
    """C++ source without its comments, trailing blanks and empty lines: an
    edit of a comment does not make a recorded measurement stale."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_hash(stage, kernel_name=""):
    """Hash of the code (comments left out) of the sources of a stage's
    kernel and the device compile flags (kernel_name: the measured kernel's
    name, which adds the sources of its own form and the flags of the
    families it is compiled in)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_nn_amd", "csrc")
    names = list(KERNEL_SOURCES[stage])
    for key, extra in KERNEL_EXTRA_SOURCES.items():
        if key in kernel_name:
            names += extra
    for n in names:
        with open(os.path.join(csrc, n)) as f:
            h.update(n.encode() + b"\0" + _code_only(f.read()).encode())
    # the device compile flags change the code as much as the sources do
    from recurrent_nn_amd import build as _build
    h.update(" ".join(_build.HIP_FLAGS).encode())
    for key, fams in KERNEL_FAMILIES.items():
        if key in kernel_name:
            for f in fams:
                if _build.FAMILY_FLAGS.get(f):
                    h.update(f"{f}:{' '.join(_build.FAMILY_FLAGS[f])}".encode())
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
    no row gather, in two operand layouts: the projection's own, X [M, K]
    times W^T with W stored [N, K] ("_xwt"; W as the operator stores it), and
    B stored [K, N].  The products write their input type (bf16 for the bf16
    ones), where the projection writes fp32 XW.  Context only: nothing on the
    measured path uses them."""
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
        del b
        w = torch.randn(N, K, device=dev, generator=g).to(dt)      # [N, K], as W is stored
        ms = ms_per(lambda: torch.mm(a, w.t()), 5)
        out[name.replace("_tflops", "_xwt_tflops")] = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        del a, w
    out["spec"] = {"hbm_gbs": HBM_PEAK_GBS, "fp32_mfma_tflops": FP32_MFMA_PEAK_TFLOPS,
                   "bf16_mfma_tflops": BF16_MFMA_PEAK_TFLOPS}
    print(json.dumps(out), flush=True)


def _pmc_rows(d, counter=False):
    """(kernel name, dispatch id, [counter name,] counter value) from every
    rocprofv3 counter csv below directory d."""
    import csv
    import glob
    rows = []
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if len(files) > 1:
        raise SystemExit(f"several counter_collection.csv under {d} (one run per directory): {files}")
    for fn in files:
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
    # "steady": the dispatches after each kernel's first one (the first runs
    # cold: instruction cache, TLB, clocks ramping up)
    def stats(v):
        ids = sorted(v)
        vals = [v[i] for i in ids]
        st = vals[1:] if len(vals) > 1 else vals
        return {"mean": float(np.mean(vals)), "first": vals[0],
                "steady_mean": float(np.mean(st)), "steady_min": float(np.min(st)),
                "steady_max": float(np.max(st)), "dispatches": len(vals)}
    out = {n: {c: stats(v) for c, v in cs.items()} for n, cs in acc.items()}
    print(json.dumps(out, indent=1))


def traffic_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, workload):
    """Per-launch HBM bytes of each kernel: mean counter KiB per dispatch over
    the steady dispatches (each kernel's first one, with cold caches and
    translation buffers, is left out when there are at least three), scaled
    by bytes / counter of the plain copy."""
    import numpy as np

    def per_kernel(d, first=None):
        acc = {}
        for name, did, v in _pmc_rows(d):
            acc.setdefault(name, {}).setdefault(did, 0.0)
            acc[name][did] += v
        out = {}
        for k, v in acc.items():
            vals = [v[i] for i in sorted(v)]
            out[k] = float(np.mean(vals[1:] if len(vals) >= 3 else vals))
            if first is not None:
                first[k] = (vals[0], len(vals))
        return out

    def copy_kib(d):
        pk = per_kernel(d)
        name = max(pk, key=pk.get)
        return name, pk[name]

    cname, cf = copy_kib(cfetch_dir)
    _, cw = copy_kib(cwrite_dir)
    rscale, wscale = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    ff, fw = {}, {}
    fk, wk = per_kernel(fetch_dir, ff), per_kernel(write_dir, fw)
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
            "first_dispatch_fetch_kib": ff[n][0], "first_dispatch_write_kib": fw.get(n, (None,))[0],
            "dispatches": ff[n][1],
            "traffic_bytes": f_kib * 1024.0 * rscale + w_kib * 1024.0 * wscale,
            "source_hash": kernel_hash(stage, n)}
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
    if k.get("source_hash") != kernel_hash(stage, k.get("name", "")):
        return None
    return k["traffic_bytes"]


def flops_per_run(c):
    """Algorithmic FLOPs of the two products of one invocation, as
    (projection, recurrence) for the nominal work (every step of every row)
    and for the valid work (D * sum(len_b) steps: positions past a row's
    length are never computed by the method; without sequence_lens the two
    are equal).  GRU lbr=0's two products per step have the same total as one
    G*H-wide product."""
    D, G = c.dirs, c.gates
    nominal_steps = c.seq * c.batch * D
    valid_steps = c.valid_cell_updates()
    per_proj = 2.0 * G * c.hidden * c.input
    per_rec = 2.0 * G * c.hidden * c.hidden
    return {"nominal": (per_proj * nominal_steps, per_rec * nominal_steps),
            "valid": (per_proj * valid_steps, per_rec * valid_steps)}


def host_facts():
    """The host's CPU model and counts (the CPU baseline's context)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(), "affinity_cpus": aff}


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
    hf = host_facts()
    return {"value": cells * reps / dt, "unit": "cell-updates/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole workload ({c.batch} rows x {c.seq} steps x {c.dirs} directions "
                      f"= {cells} cell-updates) run {reps} time(s) in {dt:.1f} s on {nt} threads",
            "threads": nt, **hf, "seconds": dt}


def measure(c, steps, warmup, dev, kernel_path=0, exact=False, time_chunk=0, stage_runs=None,
            fuse_projection=0):
    """Run one workload on the GPU: warm-up, exactly `steps` invocations
    between two events on the stream (the timed region), per-stage durations
    from the library's own events over further runs, and each invocation
    between its own events (median, minimum).  Inputs are resident in device
    memory before the timed region starts.  The plan is released before
    returning."""
    import numpy as np
    import torch

    import recurrent_nn_amd as ra

    t = {k: (v.to(dev) if v is not None and k != "sequence_lens" else v)
         for k, v in c.tensors().items()}
    stream = torch.cuda.current_stream(dev)
    with ra.plan_for_case(c, kernel_path=kernel_path, exact=exact, time_chunk=time_chunk,
                          fuse_projection=fuse_projection) as plan:
        Y = torch.empty(plan.output_shapes()[0], dtype=torch.float32, device=dev)
        Yh = torch.empty(plan.output_shapes()[1], dtype=torch.float32, device=dev)
        Yc = torch.empty_like(Yh) if c.op == "LSTM" else None
        out = (Y, Yh, Yc)

        def step():
            plan.run(t["X"], t["W"], t["R"], t["B"], t["sequence_lens"], t["initial_h"],
                     t["initial_c"], t["P"], out=out, stream=stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        plan.check(stream)
        desc = plan.describe()
        print(f"[bench] {c.name}: {desc}", file=sys.stderr, flush=True)

        # ---- the timed region: exactly `steps` invocations ------------------
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / steps
        print(f"[bench] {c.name}: {steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s)",
              file=sys.stderr, flush=True)

        # ---- per-stage durations from HIP events on the library's stream -----
        plan.enable_timing(True)
        per = {k: [] for k in ra.STAGES}
        for _ in range(stage_runs if stage_runs else max(3, steps)):
            step()
            for k, v in plan.last_timings().items():
                per[k].append(v)
        plan.enable_timing(False)
        torch.cuda.synchronize()
        plan.check(stream)
        stage_ms = {k: float(np.mean(v)) for k, v in per.items()}

        # ---- each invocation between its own events --------------------------
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a_, b_ in evs:
            a_.record(stream)
            step()
            b_.record(stream)
        torch.cuda.synchronize()
        each = sorted(a_.elapsed_time(b_) for a_, b_ in evs)
    del t, out, Y, Yh, Yc
    return {"ms": ms, "wall_s": wall, "stage_ms": stage_ms, "median": each[len(each) // 2],
            "min": each[0], "plan": desc}


def plan_fused(m):
    """Whether the measured plan computes the projection inside the step loop."""
    return "fused=1" in m["plan"].split()


def kernel_figures(c, m, exact=False):
    """Roofline figures of the projection and the step loop of one measured
    workload: achieved TFLOP/s and the fraction of the peak for the valid work
    (what the method computes) and for the nominal work (every step of every
    row).  A fused plan runs both products in the step loop: its figures
    count both, and the projection has no launch of its own."""
    fl = flops_per_run(c)
    if plan_fused(m):
        fl = {k: (0.0, v[0] + v[1]) for k, v in fl.items()}
    proj_peak = BF16_MFMA_PEAK_TFLOPS if c.proj_bf16 else FP32_MFMA_PEAK_TFLOPS
    rec_peak = FP32_MFMA_PEAK_TFLOPS
    bound = "mfma"
    if exact:
        proj_peak = rec_peak = FP32_VALU_MULADD_PEAK_TFLOPS
        bound = "alu"
    out = {}
    for i, (k, peak) in enumerate((("projection", proj_peak), ("recurrence", rec_peak))):
        ms = m["stage_ms"][k]
        fv, fn = fl["valid"][i], fl["nominal"][i]
        if plan_fused(m) and k == "projection":
            out[k] = {"fused": True, "ms": ms,
                      "note": "computed inside the step loop (its FLOPs are counted there)"}
            continue
        out[k] = {"bound": bound, "ms": ms, "peak": peak, "unit": "TFLOP/s",
                  "flop_valid": fv, "flop_nominal": fn,
                  "achieved": fv / (ms * 1e-3) / 1e12,
                  "frac": fv / (ms * 1e-3) / 1e12 / peak,
                  "achieved_nominal": fn / (ms * 1e-3) / 1e12,
                  "frac_nominal": fn / (ms * 1e-3) / 1e12 / peak}
    out["recurrence"]["us_per_step"] = m["stage_ms"]["recurrence"] * 1e3 / c.seq
    if plan_fused(m):
        out["recurrence"]["products"] = "projection + recurrent product (fused)"
    return out


def rounded(d):
    if isinstance(d, dict):
        return {k: rounded(v) for k, v in d.items()}
    if isinstance(d, float):
        return float(f"{d:.6g}")
    return d


STAMP_SLOTS, STAMP_EVENTS = 1024, 8       # recurrent_nn_amd/csrc/common.h


def step_stamps(c, dev, kernel_path=0, fuse_projection=0):
    """Cycle stamps of the instrumented build: for the two-half kernel each
    slot is a half-step (events: 0 half start, 1 product start after the flag
    wait and the first loads, 2 products issued, 3 partial tiles visible after
    the barrier, 4 gate arithmetic and stores issued, 5 this half's flag
    stored, from inside the next product); for the four-wave kernel each slot
    is a phase (0 start, 1 products issued, 2 partial tiles visible, 3 gate
    arithmetic and stores issued, 4 next phase's flags seen).  With the
    projection inside (fused), 5 is this half's flag stored from inside the
    half's share of the next step's projections and 6 the end of that
    share."""
    import numpy as np
    import torch

    import recurrent_nn_amd as ra

    t = {k: (v.to(dev) if v is not None and k != "sequence_lens" else v)
         for k, v in c.tensors().items()}
    with ra.plan_for_case(c, kernel_path=kernel_path, fuse_projection=fuse_projection) as plan:
        desc = dict(kv.split("=", 1) for kv in plan.describe().split() if "=" in kv)
        off = int(desc.get("stamps", "0"))
        if not off:
            raise SystemExit("--stamps needs the instrumented library (RNN_AMD_LIB=..._stamps.so)")
        nb = STAMP_SLOTS * STAMP_EVENTS * 8
        args = (t["X"], t["W"], t["R"], t["B"], t["sequence_lens"], t["initial_h"],
                t["initial_c"], t["P"])
        for _ in range(2):
            plan.run(*args)
        torch.cuda.synchronize()
        ws = plan.workspace(dev)
        ws[off:off + nb].zero_()
        plan.enable_timing(True)
        plan.run(*args)
        torch.cuda.synchronize()
        rec_ms = plan.last_timings()["recurrence"]
        st = ws[off:off + nb].cpu().numpy().view(np.uint64).reshape(STAMP_SLOTS, STAMP_EVENTS)
        st = st.astype(np.int64)
        halves = desc["halves"] == "2"
        fused = desc.get("fused") == "1"
        per_step = 2 if halves else int(desc["phases"])
        n = min(STAMP_SLOTS, c.seq * per_step)
        lo, hi = 2 * per_step, n - 2 * per_step          # steady slots
        rows = st[lo:hi]
        nxt = st[lo + 1:hi + 1, 0]
        names = (["wait_and_first_loads", "product", "partials_barrier", "gates_and_stores",
                  "projection_share", "barrier_to_next_half"] if fused else
                 ["wait_and_first_loads", "product", "partials_barrier", "gates_and_stores",
                  "to_next_half"] if halves else
                 ["product", "partials_barrier", "gates_and_stores", "handover_wait"])
        if fused:
            # (event 5: this half's flag stored, from inside the projection
            # share; 6: the share done)
            iv = [rows[:, 1] - rows[:, 0], rows[:, 2] - rows[:, 1], rows[:, 3] - rows[:, 2],
                  rows[:, 4] - rows[:, 3], rows[:, 6] - rows[:, 4], nxt - rows[:, 6]]
            flag = rows[:, 5] - rows[:, 4]
        elif halves:
            iv = [rows[:, 1] - rows[:, 0], rows[:, 2] - rows[:, 1], rows[:, 3] - rows[:, 2],
                  rows[:, 4] - rows[:, 3], nxt - rows[:, 4]]
            flag = rows[:, 5] - rows[:, 4]
        else:
            iv = [rows[:, 1] - rows[:, 0], rows[:, 2] - rows[:, 1], rows[:, 3] - rows[:, 2],
                  rows[:, 4] - rows[:, 3]]
        period = nxt - rows[:, 0]
        out = {"workload": c.name, "plan": plan.describe(), "workgroup": int(os.environ.get(
                   "RNN_AMD_STAMP_WG", "0")), "slot": "half-step" if halves else "phase",
               "slots_used": int(hi - lo), "recurrence_ms": rec_ms,
               "us_per_slot": rec_ms * 1e3 / (c.seq * per_step),
               "median_cycles": {k: float(np.median(v)) for k, v in zip(names, iv)},
               "median_period_cycles": float(np.median(period))}
        if halves:
            out["median_cycles"]["gates_done_to_flag_stored"] = float(np.median(flag))
        out["cycles_per_us"] = out["median_period_cycles"] / out["us_per_slot"]
    return out


# The five workloads of the operator's benchmark list; the first is timed as
# the headline line, the others are reported under "configs".
CONFIGS = ["lstm_bidir_s512_b64_i1024_h1024", "rnn_fwd_s4_b2_i3_h5", "lstm_bidir_s16_b4_i32_h64",
           "gru_fwd_s128_b32_i256_h512_lbr0", "gru_fwd_s128_b32_i256_h512_lbr1",
           "gru_rev_s256_b256_i2048_h2048_bf16"]


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, workload=args.workload)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1 "
                                   "(the multi-GPU layout is a design, not an implementation)"}))
        sys.exit(2)
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
    if args.stamps:
        torch.cuda.set_device(0)
        print(json.dumps(step_stamps(workloads.workload(args.workload), torch.device("cuda:0"),
                                     args.kernel_path, args.fuse_projection)), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = workloads.workload(args.workload)
    print(f"[bench] workload {c.name}: inputs drawn", file=sys.stderr, flush=True)
    m = measure(c, args.steps, args.warmup, dev, kernel_path=args.kernel_path, exact=args.exact,
                time_chunk=args.time_chunk, fuse_projection=args.fuse_projection)
    print(f"[bench] stage ms: {json.dumps(m['stage_ms'])}", file=sys.stderr, flush=True)
    kernels = kernel_figures(c, m, exact=args.exact)
    # size-derived rates of the step loop's operand streams (sizes over the
    # step time; not counter readings): R bytes per step (what a kernel that
    # streamed R would need from HBM) and the H rows every workgroup reads
    desc = dict(kv.split("=", 1) for kv in m["plan"].split() if "=" in kv)
    t_step = m["stage_ms"]["recurrence"] * 1e-3 / c.seq
    r_bytes = 4.0 * c.dirs * c.gates * c.hidden * c.hidden
    h_bytes = 4.0 * int(desc["workgroups"]) * int(desc["BT"]) * int(desc["Hp"])
    kernels["recurrence"]["size_derived"] = {
        "note": "operand bytes per step divided by the step time; not counter readings",
        "r_bytes_per_step": r_bytes, "r_gbs": r_bytes / t_step / 1e9,
        "r_frac_of_hbm": r_bytes / t_step / (HBM_PEAK_GBS * 1e9),
        "h_rows_read_bytes_per_step": h_bytes, "h_rows_read_gbs": h_bytes / t_step / 1e9}
    dom = "recurrence" if plan_fused(m) else max(("projection", "recurrence"),
                                                 key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    roofline = {"bound": dk["bound"], "achieved": round(dk["achieved"], 3), "peak": dk["peak"],
                "unit": dk["unit"], "frac": round(dk["frac"], 4),
                # (the recorded counters are those of the separate kernels)
                "traffic": None if plan_fused(m) else measured_traffic(c.name, dom), "kernel": dom,
                "work": "valid (sum of sequence lengths x directions steps)"}

    ms = m["ms"]
    cells = c.cell_updates()
    value = cells / (ms * 1e-3)
    res = {
        "metric": METRIC, "value": value, "unit": "cell-updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+f32" if c.proj_bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": c.name, "mode": "exact" if args.exact else "fast",
                   "time_chunk": args.time_chunk, "fuse_projection": args.fuse_projection,
                   "op": c.op, "direction": c.direction, "seq": c.seq,
                   "batch": c.batch, "input": c.input, "hidden": c.hidden, "dirs": c.dirs,
                   "layout": c.layout, "global_batch": c.batch, "seq_len": c.seq,
                   "parallelism": "none (1 GPU)", "plan": m["plan"]},
        "valid_cell_updates_per_s": c.valid_cell_updates() / (ms * 1e-3),
        "ms_per_step_median": m["median"], "ms_per_step_min": m["min"],
        "inputs_sha256": c.digests(),
        "roofline": roofline,
        "kernels": rounded(kernels),
        "stage_ms": m["stage_ms"],
    }
    del c
    # ---- the other workloads of the list, same protocol, fewer runs ---------
    if not args.no_configs and not args.exact and not args.time_chunk and not args.fuse_projection:
        confs = {}
        for name in CONFIGS:
            if name == args.workload:
                continue
            cc = workloads.workload(name)
            steps_c = max(5, min(args.steps, 20))
            mc = measure(cc, steps_c, 3, dev)
            kc = kernel_figures(cc, mc)
            confs[name] = rounded({
                "ms_per_step": mc["ms"], "ms_median": mc["median"], "ms_min": mc["min"],
                "cell_updates_per_s": cc.cell_updates() / (mc["ms"] * 1e-3),
                "valid_cell_updates_per_s": cc.valid_cell_updates() / (mc["ms"] * 1e-3),
                "steps": steps_c, "stage_ms": mc["stage_ms"], "kernels": kc, "plan": mc["plan"],
                "inputs_sha256": cc.digests()})
            del cc
        res["configs"] = confs
    if not args.no_cpu_baseline and args.cpu_budget_s > 0:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(workloads.workload(args.workload), args.cpu_budget_s)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                  "threads", "cpu_model", "host_logical_cpus",
                                                  "affinity_cpus")}
        res["gpu_over_cpu_baseline"] = value / cb["value"]
    torch.cuda.synchronize()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

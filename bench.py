#!/usr/bin/env python3
"""Benchmark of libdwc on one MI355X.

One step = one pass of the whole DWC path over one batch of the CNN-stage
workload (N=64, 56x56, C=128, 7x7 filter, pad 3, fp32, synthetic inputs):
forward at stride 1, forward at stride 2 on the same input, data gradient and
filter gradient at stride 1.  ``value`` is the nominal GFLOP/s of the step
(2*N*OH*OW*C*FH*FW per operation, the numerator of the pages' intensity
bound).  The JSON line also carries the roofline of the dominant kernel and
the CPU oracle's rate on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --copy-calibration  (a plain 256 MiB device copy, for counters)
       python bench.py --sweep OUT.jsonl [--only WORKLOAD]
                                           (every named workload, one line per op)
       python bench.py --summarize-profile DIR
           (turn the rocprofv3 CSV output of this benchmark under DIR -- trace/,
            fetch/, write/, copyf/, copyw/ and the traced run's stdout trace.log,
            made by the commands in profiles/README.md -- into profiles/*.md and
            profiles/traffic.json)
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dwc_inputs import WORKLOADS, Shape, make_inputs  # noqa: E402

METRIC = "DWC fwd/dgrad/wgrad GFLOP/s + % of roofline (HBM×η_D vs FP32/MFMA peak)"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_FP32_VECTOR = 157.3e12
PEAK_BF16_MFMA = 2.5e15
PEAK_FP8_MFMA = 5.0e15     # dense fp8 MFMA
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "e4m3": 3, "e5m2": 4}
ROTATE_BYTES = 1 << 30     # buffer sets rotate over >= 1 GiB: no Infinity-Cache reuse
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["depthwise_convolution_dwc_amd/csrc/dwc_kernels.h",
                  "depthwise_convolution_dwc_amd/csrc/dwc_plan.cpp",
                  "depthwise_convolution_dwc_amd/csrc/inst_direct.hip",
                  "depthwise_convolution_dwc_amd/csrc/inst_generic.hip"]


def kernel_source_hash() -> str:
    """Hash of the sources that decide which kernels run and what they do;
    stored counter data is only used while it matches."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- model ----

def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1, "e5m2": 1}[dtype]


def valid_taps(size_in, size_out, f, s, p):
    """sum over outputs of the number of taps that land inside the input."""
    tot = 0
    for o in range(size_out):
        lo = max(0, p - o * s)
        hi = min(f, size_in + p - o * s)
        tot += max(0, hi - lo)
    return tot


def op_model(s: Shape, op: str, dtype: str) -> dict:
    """Algorithmic FLOPs and bytes of one operation.

    F_nom = 2*N*OH*OW*C*FH*FW; the intensity bound eta_D (Flash-DWC, TACO,
    §2.2) divides it by the elements of the operation's two operands.  The
    algorithmic HBM bytes also count the fp32 output once.
    """
    nx = s.n * s.h * s.w * s.c
    ny = s.n * s.oh * s.ow * s.c
    nw = s.fh * s.fw * s.c
    eb = elem_bytes(dtype)
    f_nom = 2.0 * ny * s.fh * s.fw
    f_valid = 2.0 * s.n * s.c * valid_taps(s.h, s.oh, s.fh, s.stride_h, s.pad_h) * \
        valid_taps(s.w, s.ow, s.fw, s.stride_w, s.pad_w)
    if op == "fwd":
        operands, out = nx + nw, ny
    elif op == "bwd_data":
        operands, out = ny + nw, nx
    else:
        operands, out = nx + ny, nw
    eta = f_nom / operands
    bytes_operands = eb * operands
    bytes_alg = bytes_operands + 4 * out
    peak = {"f32": PEAK_FP32_VECTOR, "bf16": PEAK_BF16_MFMA, "f16": PEAK_BF16_MFMA,
            "e4m3": PEAK_FP8_MFMA, "e5m2": PEAK_FP8_MFMA}[dtype]
    r_lit = min(PEAK_HBM * eta / eb, peak)
    return dict(flops=f_nom, flops_valid=f_valid, eta_d=eta, bytes_operands=bytes_operands,
                bytes=bytes_alg, peak=peak, roofline=r_lit,
                bound=("hbm" if PEAK_HBM * eta / eb < peak else
                       ("alu" if dtype == "f32" else "mfma")))


def stored_traffic(kernel_names):
    """HBM bytes per launch of the named kernels from profiles/traffic.json,
    or None if absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    total = 0.0
    for k in kernel_names:
        if k not in t["kernels"]:
            return None
        total += t["kernels"][k]["bytes_per_launch"]
    return total


def roofline_entry(m: dict, seconds: float, traffic=None) -> dict:
    if m["bound"] == "hbm":
        achieved = m["bytes"] / seconds / 1e9
        peak = PEAK_HBM / 1e9
        unit = "GB/s"
    else:
        achieved = m["flops"] / seconds / 1e12
        peak = m["peak"] / 1e12
        unit = "TFLOP/s"
    return {"bound": m["bound"], "achieved": round(achieved, 3), "peak": round(peak, 3),
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic}


# --------------------------------------------------------------- device -----

def upload(op, torch, dev):
    if op.dtype == "bf16":
        return torch.from_numpy(op.stored.view(np.int16)).to(dev).view(torch.bfloat16)
    if op.dtype in ("e4m3", "e5m2"):
        tdt = torch.float8_e4m3fn if op.dtype == "e4m3" else torch.float8_e5m2
        return torch.from_numpy(op.stored).to(dev).view(tdt)
    return torch.from_numpy(op.stored).to(dev)


class OpCall:
    """One library call on preallocated buffers."""

    def __init__(self, dwc, torch, s: Shape, op: str, bufs: dict, algo: str = "auto"):
        self.s, self.op, self.b, self.algo = s, op, bufs, algo
        self.dwc, self.torch = dwc, torch
        stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
        self.stride, self.pad = stride, pad
        dev = bufs["x"].device
        if op == "fwd":
            self.out = torch.empty(s.y_shape(), dtype=torch.float32, device=dev)
        elif op == "bwd_data":
            self.out = torch.empty(s.x_shape(), dtype=torch.float32, device=dev)
        else:
            self.out = torch.empty(s.w_shape(), dtype=torch.float32, device=dev)
            p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, stride, pad, bufs["x"].dtype, algo)
            need = dwc.workspace_size(p)
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def __call__(self):
        b, s = self.b, self.s
        if self.op == "fwd":
            self.dwc.fwd(b["x"], b["w"], self.stride, self.pad, out=self.out, algo=self.algo)
        elif self.op == "bwd_data":
            self.dwc.bwd_data(b["dy"], b["w"], (s.h, s.w), self.stride, self.pad, out=self.out,
                              algo=self.algo)
        else:
            self.dwc.bwd_filter(b["x"], b["dy"], (s.fh, s.fw), self.stride, self.pad,
                                out=self.out, workspace=self.ws, algo=self.algo)


def time_step(torch, calls_per_set, steps, warmup):
    """Warm up, then time exactly `steps` steps between two events on the
    current stream, with nothing recorded between the ops (an event between
    kernels adds a few microseconds of GPU time).  Returns ms per step."""
    nsets = len(calls_per_set)
    for i in range(warmup):
        for c in calls_per_set[i % nsets]:
            c()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        for c in calls_per_set[i % nsets]:
            c()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_ops(torch, calls_per_set, reps):
    """Mean GPU duration of each op of the step: `reps` back-to-back launches
    of that op alone, each on the next buffer set (so none reads cached
    data), between two events on the stream the library launches on."""
    nsets = len(calls_per_set)
    per_op = []
    for j in range(len(calls_per_set[0])):
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(reps):
            calls_per_set[i % nsets][j]()
        end.record()
        torch.cuda.synchronize()
        per_op.append(start.elapsed_time(end) / reps)
    return per_op


# ---------------------------------------------------------- CPU oracle ------

def cpu_baseline(inp, plan, budget_s=12.0):
    """The oracle on the first n images of the batch, n sized for ~budget_s
    of CPU work; returns the nominal GFLOP/s it reaches."""
    import oracle

    x = np.ascontiguousarray(inp.x.values, dtype=np.float64)
    w = np.ascontiguousarray(inp.w.values, dtype=np.float64)
    dy_by_stride = {}

    def run(n):
        t = 0.0
        flops = 0.0
        for (s, op) in plan:
            sub = Shape(n, s.h, s.w, s.c, s.fh, s.fw, s.stride_h, s.stride_w, s.pad_h, s.pad_w)
            st, pd = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
            key = (s.oh, s.ow)
            if key not in dy_by_stride:
                dy_by_stride[key] = np.ascontiguousarray(inp.dy.values[:, :s.oh, :s.ow],
                                                         dtype=np.float64)
            dy = dy_by_stride[key][:n]
            t0 = time.perf_counter()
            if op == "fwd":
                oracle.fwd(x[:n], w, st, pd)
            elif op == "bwd_data":
                oracle.bwd_data(dy, w, (s.h, s.w), st, pd)
            else:
                oracle.bwd_filter(x[:n], dy, (s.fh, s.fw), st, pd)
            t += time.perf_counter() - t0
            flops += op_model(sub, op, inp.dtype)["flops"]
        return t, flops

    t1, _ = run(1)
    n = int(max(1, min(inp.shape.n, round(budget_s / max(t1, 1e-3)))))
    t, flops, reps = 0.0, 0.0, 0
    while t < budget_s or reps == 0:  # whole passes until the budget is spent
        dt, df = run(n)
        t, flops, reps = t + dt, flops + df, reps + 1
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(flops / t / 1e9, 3), "unit": "GFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"the same step on the first {n} of {inp.shape.n} images, {reps} passes, "
                      f"float64 on the host, {t:.1f} s"}


# ------------------------------------------------------------------ main ----

HEADLINE = "fwd_n64_56x56_c128_k7"


def kernels_of(dwc, s, op):
    """Short names of the kernels one library call launches (from its plan)."""
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w), (s.pad_h, s.pad_w))
    d = dwc.plan_describe(p, {"fwd": 0, "bwd_data": 1, "bwd_filter": 2}[op])
    fam = d.split()[1]  # sweep / direct / generic
    base = {("fwd", "sweep"): "fwd_sweep", ("bwd_data", "sweep"): "fwd_sweep",
            ("bwd_filter", "sweep"): "wgrad_sweep", ("fwd", "direct"): "fwd_rows",
            ("bwd_data", "direct"): "fwd_rows", ("bwd_filter", "direct"): "wgrad_rows",
            ("fwd", "mfma"): "fwd_mfma", ("bwd_data", "mfma"): "fwd_mfma",
            ("bwd_filter", "mfma"): "wgrad_mfma"}
    k = [base.get((op, fam), fam)]
    if op == "bwd_filter" and "ws_bytes=0" not in d:
        k.append("reduce_partials")
    return k


def headline_plan():
    s1, s2 = WORKLOADS[HEADLINE]["shapes"]
    return [(s1, "fwd"), (s2, "fwd"), (s1, "bwd_data"), (s1, "bwd_filter")]


def rotation_sets(plan, dtype) -> int:
    """Buffer sets for `plan`: the smallest op's algorithmic bytes times the
    set count reach ROTATE_BYTES (at most 16 sets)."""
    op_bytes = min(op_model(s, op, dtype)["bytes"] for s, op in plan)
    return max(1, min(16, -(-ROTATE_BYTES // max(1, int(op_bytes)))))


def build_sets(dwc, torch, plan, inp, dev, algo="auto"):
    """Enough buffer sets (each a full copy of the operands) that every op of
    the plan, run alone on consecutive sets, rotates over ROTATE_BYTES: no
    launch reads data an earlier launch left in the caches, in the step loop
    or in the per-op pass."""
    nsets = rotation_sets(plan, inp.dtype)
    host = {"x": inp.x, "w": inp.w, "dy": inp.dy}
    sets = []
    for _ in range(nsets):
        bufs = {k: upload(v, torch, dev) for k, v in host.items()}
        calls = []
        for s, op in plan:
            b = dict(bufs)
            if op != "fwd" and (s.oh, s.ow) != tuple(bufs["dy"].shape[1:3]):
                b["dy"] = bufs["dy"][:, :s.oh, :s.ow].contiguous()
            calls.append(OpCall(dwc, torch, s, op, b, algo))
        sets.append(calls)
    return sets


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--sweep", default=None, help="write per-op lines of every workload here")
    ap.add_argument("--only", default=None, metavar="WORKLOAD",
                    help="with --sweep: only this named workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 256 MiB a few times (scales the byte counters)")
    ap.add_argument("--summarize-profile", default=None, metavar="DIR",
                    help="write profiles/ from the rocprofv3 output under DIR")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        x = torch.randn(64 * 1024 * 1024, device="cuda")  # 256 MiB
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print("copied 256 MiB 5 times", flush=True)
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this DWC library runs on a single device)", file=sys.stderr)
        sys.exit(2)

    import torch

    import depthwise_convolution_dwc_amd as dwc

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    dwc.lib()

    if args.sweep:
        return sweep(dwc, torch, dev, args)

    plan = headline_plan()
    wl = WORKLOADS[HEADLINE]
    s1 = plan[0][0]
    inp = make_inputs(s1, "f32", seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
    sets = build_sets(dwc, torch, plan, inp, dev)
    log(f"bench: {len(sets)} buffer sets, {args.warmup} warmup + {args.steps} timed steps")
    ms = time_step(torch, sets, args.steps, args.warmup)
    per_op = time_ops(torch, sets, args.steps)

    models = [op_model(s, op, "f32") for s, op in plan]
    flops = sum(m["flops"] for m in models)
    names = ["fwd_s1", "fwd_s2", "bwd_data", "bwd_filter"]
    ops = {}
    for name, m, t in zip(names, models, per_op):
        ops[name] = {"ms": round(t, 5), "gflops": round(m["flops"] / (t * 1e-3) / 1e9, 1),
                     "roofline_frac": round(m["flops"] / (t * 1e-3) / m["roofline"], 4),
                     "bound": m["bound"]}
    dom = int(np.argmax(per_op))
    s_dom, op_dom = plan[dom]
    kern = kernels_of(dwc, s_dom, op_dom)
    roof = roofline_entry(models[dom], per_op[dom] * 1e-3, stored_traffic(kern))
    roof["kernel"] = "+".join(kern)
    roof["op"] = names[dom]
    cpu = None
    if not args.no_cpu:
        log("bench: timing the CPU oracle on a sample of the batch")
        cpu = cpu_baseline(inp, plan, args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": round(flops / (ms * 1e-3) / 1e9, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "CNN stage N=64 56x56 C=128 7x7 pad 3, fp32: "
                               "fwd stride 1 + fwd stride 2 + bwd_data + bwd_filter",
                   "n": 64, "h": 56, "w": 56, "c": 128, "filter": 7, "pad": 3,
                   "global_batch": 64, "parallelism": "single-gpu"},
        "ops": ops,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _kernel_short(name: str) -> str:
    # "void dwc::fwd_sweep<0, 7, 7, false>(dwc::SweepArgs)" -> "fwd_sweep"
    n = name.split("(")[0].replace("void ", "").replace("dwc::", "")
    return n.split("<")[0].strip()


def _csv_rows(d, pattern):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


PROFILE_STEPS, PROFILE_WARMUP = 20, 5
PROFILE_NAME = "cnn_stage_n64_56x56_c128_k7_fp32_step"
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof/trace "
             f"-o run -- python3 $R/bench.py --steps {PROFILE_STEPS} --warmup {PROFILE_WARMUP} "
             "--no-cpu > $R/gpurun_out/prof/trace.log",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/fetch -o run "
             "-- python3 $R/bench.py --steps 5 --warmup 2 --no-cpu",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/write -o run "
             "-- python3 $R/bench.py --steps 5 --warmup 2 --no-cpu",
    "copyf": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/copyf -o run "
             "-- python3 $R/bench.py --copy-calibration",
    "copyw": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/copyw -o run "
             "-- python3 $R/bench.py --copy-calibration",
}
# kernel-name prefixes: fwd_sweep<DT, F, TMW, FLIP, PROLOGUE>
OP_KERNELS = {"fwd_s1": ["fwd_sweep<0, 7, 7, false"], "fwd_s2": ["fwd_rows<0, 7, 2"],
              "bwd_data": ["fwd_sweep<0, 7, 7, true"],
              "bwd_filter": ["wgrad_sweep<0, 7, 7>", "reduce_partials"]}


def summarize_profile(d):
    """Write profiles/<workload>.kernel_trace.md, .hbm_traffic.md and
    traffic.json from the rocprofv3 output of this benchmark under d."""
    os.makedirs(PROFILES, exist_ok=True)
    cd = "cd /tmp && export TMPDIR=/tmp && "
    # kernel trace: per-kernel durations in dispatch order.  The traced run
    # launches each kernel PROFILE_WARMUP + PROFILE_STEPS times in the step
    # loop, then PROFILE_STEPS times back to back in the per-op pass that
    # gives the JSON line's per-op durations.
    rows = sorted(_csv_rows(os.path.join(d, "trace"), "*kernel_trace.csv"),
                  key=lambda r: int(r["Start_Timestamp"]))
    stats = {}
    for r in rows:
        stats.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | calls | avg us (all) | min us | max us | avg us (per-op pass) |",
             "|---|---|---|---|---|---|"]
    passavg = {}
    for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        passavg[k] = float(np.mean(v[-PROFILE_STEPS:]))
        lines.append(f"| `{k}` | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{passavg[k]:.2f} |")
    traced = None
    log_path = os.path.join(d, "trace.log")
    if os.path.exists(log_path):
        for ln in open(log_path):
            if ln.startswith("{") and '"metric"' in ln:
                traced = json.loads(ln)
    cmp = ["| op | kernels | rocprofv3 per-op pass, us | JSON line `ops.<op>.ms`, us |",
           "|---|---|---|---|"]
    for op, pats in OP_KERNELS.items():
        ks = [k for p in pats for k in stats if p in k]
        tr = sum(passavg[k] for k in ks)
        js = traced["ops"][op]["ms"] * 1e3 if traced else float("nan")
        cmp.append(f"| {op} | {' + '.join(_kernel_short(k) for k in ks)} | {tr:.2f} | {js:.2f} |")
    trace_md = f"""# Kernel trace: CNN-stage step, N=64 56x56 C=128 7x7 pad 3, fp32

One benchmark step = forward stride 1 + forward stride 2 + data gradient +
filter gradient on the same batch (the default `bench.py` workload), on one
MI355X, buffer sets rotating over >= 1 GiB (no Infinity-Cache reuse).  The
traced run launches each kernel {PROFILE_WARMUP} + {PROFILE_STEPS} times in
the step loop, then {PROFILE_STEPS} times back to back in the per-op pass
whose event timings give the JSON line's per-op durations.

Command (repository root `$R`):

```
{cd}{PROFILE_CMDS["trace"]}
cd $R && python3 bench.py --summarize-profile gpurun_out/prof
```

Durations from the dispatch timestamps of `run_kernel_trace.csv`:

{chr(10).join(lines)}

`fwd_sweep<0, 7, 7, true, ..>` is the data gradient (the forward sweep on dY with the
filter turned by 180 degrees); `fwd_rows<0, 7, 2, ...>` is the stride-2
forward; the filter gradient is `wgrad_sweep` followed by `reduce_partials`.

Per-op durations of the same traced command: the kernels' rocprofv3 average
over the per-op pass against the JSON line it printed (HIP events on the
library's stream; under the profiler both run a few percent slower than in
an unprofiled run):

{chr(10).join(cmp)}
"""
    with open(os.path.join(PROFILES, PROFILE_NAME + ".kernel_trace.md"), "w") as f:
        f.write(trace_md)

    def per_kernel(sub, counter):
        acc = {}
        for r in _csv_rows(os.path.join(d, sub), "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: float(np.mean(v)) for k, v in acc.items()}

    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    cf = per_kernel("copyf", "FETCH_SIZE")
    cw = per_kernel("copyw", "WRITE_SIZE")
    copy_bytes = 256 * 1024 * 1024  # the calibration copy moves 256 MiB each way
    ck = [k for k in cf if "copyBuffer" in k]
    f_scale = copy_bytes / cf[ck[0]] if ck else 1.0
    w_scale = copy_bytes / cw[ck[0]] if ck else 1.0
    kernels = {}
    for k in set(fetch) | set(write):
        short = _kernel_short(k)
        fb = fetch.get(k, 0.0) * f_scale
        wb = write.get(k, 0.0) * w_scale
        kernels.setdefault(short, {"fetch_bytes": 0.0, "write_bytes": 0.0, "n": 0, "names": []})
        e = kernels[short]
        e["fetch_bytes"] += fb
        e["write_bytes"] += wb
        e["n"] += 1
        e["names"].append(k)
    for e in kernels.values():
        e["fetch_bytes"] /= e["n"]
        e["write_bytes"] /= e["n"]
        e["bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
    out = {"source_hash": kernel_source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": kernels}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    tl = ["| kernel | FETCH bytes/launch | WRITE bytes/launch | total |", "|---|---|---|---|"]
    for k, e in sorted(kernels.items()):
        tl.append(f"| `{k}` | {e['fetch_bytes'] / 1e6:.1f} MB | {e['write_bytes'] / 1e6:.1f} MB | "
                  f"{e['bytes_per_launch'] / 1e6:.1f} MB |")
    cmds = "\n".join(cd + PROFILE_CMDS[k] for k in ("fetch", "write", "copyf", "copyw"))
    traffic_md = f"""# HBM traffic per launch: CNN-stage step, N=64 56x56 C=128 7x7 pad 3, fp32

Per-dispatch `FETCH_SIZE` and `WRITE_SIZE` (KiB, rocprofv3 derived counters,
each in a run of its own), averaged over the step's launches of each kernel
and scaled by what the same counters read for a plain 256 MiB device copy
(`bench.py --copy-calibration`, the runtime's copyBuffer kernel): on this
MI355X `FETCH_SIZE` reads {1 / f_scale:.3f} of the copied bytes (scale
{f_scale:.3f}) and `WRITE_SIZE` {1 / w_scale:.3f} (scale {w_scale:.3f}).

Commands (repository root `$R`):

```
{cmds}
cd $R && python3 bench.py --summarize-profile gpurun_out/prof
```

{chr(10).join(tl)}

Algorithmic bytes for comparison (each operand read once, output written
once): forward 102.8 MB in + 102.8 MB out; stride-2 forward 102.8 MB in +
25.7 MB out; filter gradient 102.8 MB (X) + 102.8 MB (dY) in.  The same
numbers are in `traffic.json`, which `bench.py` reads for the `traffic`
field of its roofline entry while the kernel sources are unchanged (their
hash is stored with the data).
"""
    with open(os.path.join(PROFILES, PROFILE_NAME + ".hbm_traffic.md"), "w") as f:
        f.write(traffic_md)
    print(trace_md)
    print(traffic_md)


def sweep(dwc, torch, dev, args):
    out = open(args.sweep, "w")
    for name, wl in WORKLOADS.items():
        if args.only and name != args.only:
            continue
        for s in wl["shapes"]:
            for dt in wl["dtypes"]:
                inp = make_inputs(s, dt, seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
                # half-precision operands: the vector kernels and the library's
                # choice (the packed-MFMA kernels where they apply) side by side
                for op, algo in [(o, a) for o in wl["ops"]
                                 for a in (("direct", "auto") if dt != "f32" else ("auto",))]:
                    plan = [(s, op)]
                    sets = build_sets(dwc, torch, plan, inp, dev, algo)
                    steps = max(10, min(args.steps, 200))
                    # ten warm-up launches right after the upload timed short
                    # kernels up to 25% slow: run the op for ~50 ms first
                    t1 = time_step(torch, sets, 3, 1)
                    warm = int(min(2000, max(args.warmup, 50.0 / max(t1, 1e-3))))
                    ms = time_step(torch, sets, steps, warm)
                    m = op_model(s, op, dt)
                    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                                    (s.pad_h, s.pad_w), DTYPE_CODE[dt], algo)
                    rec = {"workload": name, "shape": [s.n, s.h, s.w, s.c, s.fh, s.fw,
                                                       s.stride_h, s.pad_h],
                           "dtype": dt, "op": op, "algo": algo, "ms": round(ms, 5),
                           "gflops": round(m["flops"] / (ms * 1e-3) / 1e9, 1),
                           "gflops_valid": round(m["flops_valid"] / (ms * 1e-3) / 1e9, 1),
                           "valid_frac": round(m["flops_valid"] / m["flops"], 3),
                           "gbps": round(m["bytes"] / (ms * 1e-3) / 1e9, 1),
                           "roofline_tflops": round(m["roofline"] / 1e12, 2),
                           "roofline_frac": round(m["flops"] / (ms * 1e-3) / m["roofline"], 4),
                           "bound": m["bound"],
                           "plan": dwc.plan_describe(p, {"fwd": 0, "bwd_data": 1,
                                                         "bwd_filter": 2}[op])}
                    out.write(json.dumps(rec) + "\n")
                    out.flush()
                    log(json.dumps(rec))
                    del sets
                torch.cuda.empty_cache()
    out.close()


if __name__ == "__main__":
    main()

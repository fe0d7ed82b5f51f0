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
       python bench.py --sweep OUT.jsonl   (every named workload, one line per op)
"""

from __future__ import annotations

import argparse
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
ROTATE_BYTES = 1 << 30     # buffer sets rotate over >= 1 GiB: no Infinity-Cache reuse


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- model ----

def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


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
    peak = PEAK_FP32_VECTOR if dtype == "f32" else PEAK_BF16_MFMA
    r_lit = min(PEAK_HBM * eta / eb, peak)
    return dict(flops=f_nom, flops_valid=f_valid, eta_d=eta, bytes_operands=bytes_operands,
                bytes=bytes_alg, peak=peak, roofline=r_lit,
                bound=("hbm" if PEAK_HBM * eta / eb < peak else
                       ("alu" if dtype == "f32" else "mfma")))


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
    return torch.from_numpy(op.stored).to(dev)


class OpCall:
    """One library call on preallocated buffers."""

    def __init__(self, dwc, torch, s: Shape, op: str, bufs: dict):
        self.s, self.op, self.b = s, op, bufs
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
            p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, stride, pad, bufs["x"].dtype)
            need = dwc.workspace_size(p)
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def __call__(self):
        b, s = self.b, self.s
        if self.op == "fwd":
            self.dwc.fwd(b["x"], b["w"], self.stride, self.pad, out=self.out)
        elif self.op == "bwd_data":
            self.dwc.bwd_data(b["dy"], b["w"], (s.h, s.w), self.stride, self.pad, out=self.out)
        else:
            self.dwc.bwd_filter(b["x"], b["dy"], (s.fh, s.fw), self.stride, self.pad,
                                out=self.out, workspace=self.ws)


def time_step(torch, calls_per_set, steps, warmup):
    """Warm up, then time exactly `steps` steps with events between the ops.
    Returns (ms per step, per-op mean ms)."""
    nsets = len(calls_per_set)
    nops = len(calls_per_set[0])
    for i in range(warmup):
        for c in calls_per_set[i % nsets]:
            c()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nops + 1)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        calls = calls_per_set[i % nsets]
        e = evs[i]
        for j, c in enumerate(calls):
            e[j].record()
            c()
        e[nops].record()
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    per_op = [float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
              for j in range(nops)]
    return total / steps, per_op


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
    t, flops = run(n)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(flops / t / 1e9, 3), "unit": "GFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"same step on the first {n} of {inp.shape.n} images, float64, "
                      f"{t:.1f} s"}


# ------------------------------------------------------------------ main ----

HEADLINE = "fwd_n64_56x56_c128_k7"


def headline_plan():
    s1, s2 = WORKLOADS[HEADLINE]["shapes"]
    return [(s1, "fwd"), (s2, "fwd"), (s1, "bwd_data"), (s1, "bwd_filter")]


def build_sets(dwc, torch, plan, inp, dev):
    """Enough buffer sets (each a full copy of the operands) to rotate over
    ROTATE_BYTES, so no step reads a set the previous steps left in cache."""
    set_bytes = 0
    for s, op in plan:
        m = op_model(s, op, inp.dtype)
        set_bytes += m["bytes"]
    nsets = max(1, min(8, -(-ROTATE_BYTES // max(1, int(set_bytes)))))
    host = {"x": inp.x, "w": inp.w, "dy": inp.dy}
    sets = []
    for _ in range(nsets):
        bufs = {k: upload(v, torch, dev) for k, v in host.items()}
        calls = []
        for s, op in plan:
            b = dict(bufs)
            if op != "fwd" and (s.oh, s.ow) != tuple(bufs["dy"].shape[1:3]):
                b["dy"] = bufs["dy"][:, :s.oh, :s.ow].contiguous()
            calls.append(OpCall(dwc, torch, s, op, b))
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
    args = ap.parse_args()
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
    ms, per_op = time_step(torch, sets, args.steps, args.warmup)

    models = [op_model(s, op, "f32") for s, op in plan]
    flops = sum(m["flops"] for m in models)
    names = ["fwd_s1", "fwd_s2", "bwd_data", "bwd_filter"]
    ops = {}
    for name, m, t in zip(names, models, per_op):
        ops[name] = {"ms": round(t, 5), "gflops": round(m["flops"] / (t * 1e-3) / 1e9, 1),
                     "roofline_frac": round(m["flops"] / (t * 1e-3) / m["roofline"], 4),
                     "bound": m["bound"]}
    dom = int(np.argmax(per_op))
    roof = roofline_entry(models[dom], per_op[dom] * 1e-3)
    roof["kernel"] = names[dom]
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


def sweep(dwc, torch, dev, args):
    out = open(args.sweep, "w")
    for name, wl in WORKLOADS.items():
        for s in wl["shapes"]:
            for dt in wl["dtypes"]:
                inp = make_inputs(s, dt, seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
                for op in wl["ops"]:
                    plan = [(s, op)]
                    sets = build_sets(dwc, torch, plan, inp, dev)
                    steps = max(10, min(args.steps, 200))
                    ms, _ = time_step(torch, sets, steps, min(args.warmup, 10))
                    m = op_model(s, op, dt)
                    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                                    (s.pad_h, s.pad_w), {"f32": 0, "bf16": 1, "f16": 2}[dt])
                    rec = {"workload": name, "shape": [s.n, s.h, s.w, s.c, s.fh, s.fw,
                                                       s.stride_h, s.pad_h],
                           "dtype": dt, "op": op, "ms": round(ms, 5),
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

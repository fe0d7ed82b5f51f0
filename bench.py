#!/usr/bin/env python3
"""Benchmark of libdwc on one MI355X.

One step = one pass of the whole DWC path -- forward, data gradient and
filter gradient -- over one batch of the largest single-GPU workload: N=128,
28x28, C=512, 31x31 filter, pad 15, fp16 operands with fp32 accumulation and
outputs, synthetic inputs, every operation through the library's own kernel
choice (the packed-MFMA kernels here).  ``value`` is the nominal GFLOP/s of
the step (2*N*OH*OW*C*FH*FW per operation, the numerator of the pages'
intensity bound).  The JSON line also carries the roofline of the dominant
kernel, the CPU oracle's rate on a bounded sample, and per-configuration
entries (every named workload, each operation timed alone: ms and fraction
of its literal roofline), whose full records (nominal and valid GFLOP/s,
GB/s, full-traffic fraction, kernels) go to --details.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--config-reps R] [--no-configs] [--details FILE]
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

from dwc_inputs import SWEEP_FILTERS, WORKLOADS, Shape, make_inputs  # noqa: E402

METRIC = "DWC fwd/dgrad/wgrad GFLOP/s + % of roofline (HBM×η_D vs FP32/MFMA peak)"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_FP32_VECTOR = 157.3e12
PEAK_BF16_MFMA = 2.5e15
PEAK_FP8_MFMA = 5.0e15     # dense fp8 MFMA
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "e4m3": 3, "e5m2": 4}
ROTATE_BYTES = 1 << 30     # buffer sets rotate over >= 1 GiB: no Infinity-Cache reuse
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = sorted(
    os.path.join("depthwise_convolution_dwc_amd", "csrc", f)
    for f in os.listdir(os.path.join(ROOT, "depthwise_convolution_dwc_amd", "csrc"))
    if f.endswith((".h", ".hip", ".cpp")))


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


def stored_traffic(kernel_specs):
    """HBM bytes per launch of the given kernels (kernels_of() entries) from
    profiles/traffic.json, or None if absent or taken on other kernel
    sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    total = 0.0
    for spec in kernel_specs:
        ks = kernel_matches(t["kernels"], spec)
        if len(ks) != 1:
            return None
        total += t["kernels"][ks[0]]["bytes_per_launch"]
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


def time_ops_graph(torch, calls_per_set, reps):
    """time_ops() without the host: the `reps` launches of each op are
    captured once in a HIP graph (on rotating buffer sets, as above) and the
    graph is replayed between two events, so short kernels are not timed at
    the rate the host can issue them.  The graph's last output of one set
    must equal an eager launch's bit for bit (the library is deterministic).
    Returns (per-op ms, "graph"), or time_ops() and "eager" if a capture is
    refused."""
    nsets = len(calls_per_set)
    per_op = []
    try:
        for j in range(len(calls_per_set[0])):
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for i in range(reps):
                    calls_per_set[i % nsets][j]()
            g.replay()  # warm
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            g.replay()
            end.record()
            torch.cuda.synchronize()
            per_op.append(start.elapsed_time(end) / reps)
            last = calls_per_set[(reps - 1) % nsets][j]
            got = last.out.clone()
            last()
            torch.cuda.synchronize()
            if not torch.equal(got, last.out):
                raise RuntimeError("graph replay differs from an eager launch")
            del g
        return per_op, "graph"
    except RuntimeError as e:
        if "differs" in str(e):
            raise
        log(f"bench: graph capture refused ({e}); timing eager launches")
        return time_ops(torch, calls_per_set, reps), "eager"


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
            "cpu": cpu_model(), "kind": "oracle",
            "sample": f"the same step on the first {n} of {inp.shape.n} images, {reps} passes, "
                      f"float64 on the host, {t:.1f} s"}


# ------------------------------------------------------------------ main ----

HEADLINE = "mixed_n128_28x28_c512"
HEADLINE_SHAPE = 1          # the 31x31 shape of that workload
HEADLINE_DTYPE = "f16"
HEADLINE_OPS = ("fwd", "bwd_data", "bwd_filter")


def kernels_of(dwc, s, op, dtype="f32", algo="auto"):
    """The kernels one library call launches, each as 'name<template
    arguments the plan fixes|workgroups' (a prefix of the full kernel name
    in a rocprofv3 trace, and its launch size)."""
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                    (s.pad_h, s.pad_w), DTYPE_CODE[dtype], algo)
    d = dwc.plan_describe(p, {"fwd": 0, "bwd_data": 1, "bwd_filter": 2}[op])
    fam = d.split()[1]  # sweep / direct / generic / mfma / phase
    kv = dict(t.split("=", 1) for t in d.split()[2:] if "=" in t)
    dt = DTYPE_CODE[dtype]
    flip = "true" if kv.get("flip") == "1" or (op == "bwd_data" and fam in ("mfma", "sweep")) \
        else "false"
    blocks = kv.get("blocks")
    if fam == "mfma":
        if kv.get("h4") == "1":  # 16-bit 4x4x4 kernel
            k = f"fwd_mfma_h4n<{dt}, {kv['fwi']}, {kv['t']}, {flip}>"
        elif kv.get("f32") == "1":  # fp32 matrix-core kernels
            k = (f"wgrad_mfma_f32<{dt}, {kv['tw']}, {kv['nb']}>" if op == "bwd_filter" else
                 f"fwd_mfma_f32n<{kv['fwi']}, {kv['t']}, {flip}>" if kv.get('img') == '1' else
                 f"fwd_mfma_f32<{dt}, {kv['fwi']}, {kv['t']}, {flip}>")
        elif op == "bwd_filter":
            k = f"wgrad_mfma{'8' if dt >= 3 else ''}<{dt}, {kv['nfm']}, {kv['nfn']}, {kv['nk']}, " \
                f"{kv['pf']}>"
        elif kv.get("batch") == "1" and kv.get("imgs") == "16":
            k = f"fwd_mfma_batch16<{dt}, {kv['ocg']}, {flip}>"
        elif kv.get("batch") == "1":
            k = f"fwd_mfma_batch<{dt}, {kv['cb']}, {flip}>"
        elif dt >= 3:
            k = f"fwd_mfma8<{dt}, {kv['nf']}, {kv['tiles']}, {flip}>"
        else:
            k = f"fwd_mfma<{dt}, {kv['nf']}, {kv['cb']}, {kv['tiles']}, {flip}>"
    elif fam == "sweep":
        k = (f"wgrad_sweep<{dt}, {kv['f']}, {kv['strip']}>" if op == "bwd_filter" else
             f"fwd_sweep<{dt}, {kv['f']}, {kv['strip']}, {flip}")
    elif fam == "direct":
        k = (f"wgrad_rows<{dt}, {kv['kfw']}, {kv['sw']}, {kv['tj']}>" if op == "bwd_filter" else
             f"fwd_rows<{dt}, {kv['kfw']}, {kv['sw']}, {kv['tmw']}, {flip}")
    elif fam == "phase":
        k = f"dgrad_phase<{dt}, {kv['km']}, "
    else:  # generic: one lane per output, 256 per workgroup
        k = {"fwd": f"fwd_generic<{dt}, false>", "bwd_data": f"dgrad_generic<{dt}>",
             "bwd_filter": f"wgrad_generic<{dt}>"}[op]
        blocks = str(-(-int(kv["total"]) // 256))
    ks = [f"{k}|{blocks}"]
    if op == "bwd_filter" and "ws_bytes=0" not in d:
        m = s.fh * s.fw * s.c
        if int(kv.get("z", 1)) > 32:  # many slices: 16 waves split them, 64 elements a block
            ks.append(f"reduce_partials_split|{-(-m // 64)}")
        else:
            # four partial elements per thread where 16-byte accesses line up
            # (the channel-blocked partials of the packed kernels need C % 4 == 0)
            v4 = s.c % 4 == 0 if fam == "mfma" else m % 4 == 0
            ks.append(f"reduce_partials<{4 if v4 else 1}>|{-(-(m // 4 if v4 else m) // 256)}")
    return ks


def kernel_matches(keys, spec):
    """The keys ('full name|workgroups') that a kernels_of() entry names."""
    pre, blocks = spec.split("|")
    return [k for k in keys if k.split("|")[0].startswith(pre) and k.split("|")[1] == blocks]


def headline_plan():
    s = WORKLOADS[HEADLINE]["shapes"][HEADLINE_SHAPE]
    return [(s, op) for op in HEADLINE_OPS]


def rotation_sets(plan, dtype) -> int:
    """Buffer sets for `plan`: the smallest op's algorithmic bytes times the
    set count reach ROTATE_BYTES (at most 64 sets)."""
    op_bytes = min(op_model(s, op, dtype)["bytes"] for s, op in plan)
    return max(1, min(64, -(-ROTATE_BYTES // max(1, int(op_bytes)))))


def build_sets(dwc, torch, plan, inp, dev, algo="auto"):
    """Enough buffer sets (each a full copy of the operands) that every op of
    the plan, run alone on consecutive sets, rotates over ROTATE_BYTES: no
    launch reads data an earlier launch left in the caches, in the step loop
    or in the per-op pass.  The operands are uploaded once and copied on
    the device."""
    nsets = rotation_sets(plan, inp.dtype)
    first = {k: upload(v, torch, dev) for k, v in {"x": inp.x, "w": inp.w, "dy": inp.dy}.items()}
    sets = []
    for i in range(nsets):
        bufs = first if i == 0 else {k: v.clone() for k, v in first.items()}
        calls = []
        for s, op in plan:
            b = dict(bufs)
            if op != "fwd" and (s.oh, s.ow) != tuple(bufs["dy"].shape[1:3]):
                b["dy"] = bufs["dy"][:, :s.oh, :s.ow].contiguous()
            calls.append(OpCall(dwc, torch, s, op, b, algo))
        sets.append(calls)
    return sets


def config_label(name, s, dt):
    """Short key of one measured configuration."""
    tag = {"fwd_n1_14x14_c32_k7": "c1", "fwd_n64_56x56_c128_k7": "c2",
           "all_n32_56x56_c128_k31": "c3", "sweep_n64_stages": "c4",
           "mixed_n128_28x28_c512": "c5", "strided_bwd_n64_56x56_c128_k7_s2": "f1",
           "lowbit_n128_28x28_c512": "f4"}[name]
    return tag, f"{s.h}x{s.w}c{s.c}k{s.fh}s{s.stride_h}-{dt}"


def config_cases(fp8_formats=("e4m3",)):
    """(workload, shape, dtype, op, algo) of every per-configuration entry:
    all five configurations of the target (half-precision ones on the
    library's choice and on the vector kernels) and the measured "next"
    rows (strided backward; fp8 operands, e4m3 -- e5m2 runs the same
    kernels)."""
    for name, wl in WORKLOADS.items():
        for s in wl["shapes"]:
            for dt in wl["dtypes"]:
                if dt in ("e4m3", "e5m2") and dt not in fp8_formats:
                    continue
                algos = ("auto",) if dt == "f32" else ("auto", "direct")
                for op in wl["ops"]:
                    for algo in algos:
                        yield name, s, dt, op, algo


def measure_configs(dwc, torch, dev, reps, warmup_ms=50.0):
    """Every configuration entry timed alone: `reps` back-to-back launches
    on rotating buffer sets between two events, after ~warmup_ms of the
    same launches.  Returns (compact summary for the JSON line, full
    records)."""
    records = []
    groups = {}
    for case in config_cases():
        name, s, dt, op, algo = case
        groups.setdefault((name, s, dt), []).append((op, algo))
    for (name, s, dt), ops in groups.items():
        wl = WORKLOADS[name]
        inp = make_inputs(s, dt, seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
        for algo in sorted({a for _, a in ops}):
            plan = [(s, op) for op, a in ops if a == algo]
            sets = build_sets(dwc, torch, plan, inp, dev, algo)
            t1 = time_ops(torch, sets, 3)
            warm = max(int(min(2000, max(5, warmup_ms / max(t, 1e-3)))) for t in t1)
            time_ops(torch, sets, warm)
            per_op, how = time_ops_graph(torch, sets, reps)
            for (s_, op), ms in zip(plan, per_op):
                m = op_model(s_, op, dt)
                tag, key = config_label(name, s_, dt)
                full_peak = min(PEAK_HBM * m["flops"] / m["bytes"], m["peak"])
                records.append({
                    "config": tag, "workload": name, "case": key, "op": op, "algo": algo,
                    "kernels": "+".join(kernels_of(dwc, s_, op, dt, algo)),
                    "ms": round(ms, 5),
                    "gflops": round(m["flops"] / (ms * 1e-3) / 1e9, 1),
                    "gflops_valid": round(m["flops_valid"] / (ms * 1e-3) / 1e9, 1),
                    "valid_frac": round(m["flops_valid"] / m["flops"], 3),
                    "gbps": round(m["bytes"] / (ms * 1e-3) / 1e9, 1),
                    "roofline_frac": round(m["flops"] / (ms * 1e-3) / m["roofline"], 4),
                    "full_traffic_frac": round(m["flops"] / (ms * 1e-3) / full_peak, 4),
                    "bound": m["bound"], "warm": warm, "reps": reps, "timing": how})
            log(f"bench: {name} {key} {algo}: " +
                ", ".join(f"{r['op']} {r['ms'] * 1e3:.1f} us" for r in records[-len(plan):]))
            del sets
        torch.cuda.empty_cache()
    return compact_configs(records), records


def compact_configs(records):
    """The per-configuration entries of the JSON line: for each
    configuration and case, op -> [microseconds, fraction of the literal
    roofline]; half-precision cases also on the vector kernels (op@vector);
    the 36-point filter sweep as per-stage lists over its nine filters.  The
    fp8 row's vector-kernel times stay in the detail records only."""
    out = {}
    for r in records:
        if r["algo"] != "auto" and r["config"] == "f4":
            continue
        op = r["op"] + ("" if r["algo"] == "auto" else "@vector")
        us, fr = round(r["ms"] * 1e3, 1), round(r["roofline_frac"], 3)
        if r["config"] == "c4":
            stage, f = r["case"].split("k")[0], int(r["case"].split("k")[1].split("s")[0])
            d = out.setdefault("c4", {"filters": list(SWEEP_FILTERS)}).setdefault(stage, {})
            d.setdefault(op + ".us", []).append(us)
            d.setdefault(op + ".frac", []).append(fr)
            assert SWEEP_FILTERS[len(d[op + ".us"]) - 1] == f
        else:
            out.setdefault(r["config"], {}).setdefault(r["case"], {})[op] = [us, fr]
    return out


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--config-reps", type=int, default=500,
                    help="launches per timed per-configuration entry")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration entries")
    ap.add_argument("--details", default=None,
                    help="write the full per-configuration records here (JSON lines)")
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
    dt = HEADLINE_DTYPE
    inp = make_inputs(s1, dt, seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
    sets = build_sets(dwc, torch, plan, inp, dev)
    log(f"bench: {len(sets)} buffer sets, {args.warmup} warmup + {args.steps} timed steps")
    ms = time_step(torch, sets, args.steps, args.warmup)
    per_op = time_ops(torch, sets, args.steps)
    del sets
    torch.cuda.empty_cache()

    models = [op_model(s, op, dt) for s, op in plan]
    flops = sum(m["flops"] for m in models)
    ops = {}
    for (s, op), m, t in zip(plan, models, per_op):
        ops[op] = {"ms": round(t, 5), "gflops": round(m["flops"] / (t * 1e-3) / 1e9, 1),
                   "roofline_frac": round(m["flops"] / (t * 1e-3) / m["roofline"], 4),
                   "bound": m["bound"]}
    dom = int(np.argmax(per_op))
    s_dom, op_dom = plan[dom]
    kern = kernels_of(dwc, s_dom, op_dom, dt)
    roof = roofline_entry(models[dom], per_op[dom] * 1e-3, stored_traffic(kern))
    roof["kernel"] = "+".join(kern)
    roof["op"] = op_dom
    configs = None
    if not args.no_configs:
        log(f"bench: per-configuration entries, {args.config_reps} launches each")
        configs, records = measure_configs(dwc, torch, dev, args.config_reps)
        if args.details:
            with open(args.details, "w") as f:
                for r in records:
                    f.write(json.dumps(r) + "\n")
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
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": "mixed precision N=128 28x28 C=512 31x31 pad 15, fp16 operands, "
                               "fp32 accumulation and outputs: fwd + bwd_data + bwd_filter",
                   "n": 128, "h": 28, "w": 28, "c": 512, "filter": 31, "pad": 15,
                   "global_batch": 128, "parallelism": "single-gpu"},
        "ops": ops,
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(line, separators=(",", ":")), flush=True)


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


PROFILE_STEPS, PROFILE_WARMUP, PROFILE_REPS = 20, 5, 20
PROFILE_NAME = "mixed_n128_28x28_c512_k31_f16_step"
_BENCH = "python3 $R/bench.py --no-cpu"
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof/trace "
             f"-o run -- {_BENCH} --steps {PROFILE_STEPS} --warmup {PROFILE_WARMUP} "
             f"--config-reps {PROFILE_REPS} --details $R/gpurun_out/prof/details.jsonl "
             "> $R/gpurun_out/prof/trace.log",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/fetch -o run "
             f"-- {_BENCH} --steps 5 --warmup 2 --config-reps 5",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/write -o run "
             f"-- {_BENCH} --steps 5 --warmup 2 --config-reps 5",
    "copyf": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/copyf -o run "
             "-- python3 $R/bench.py --copy-calibration",
    "copyw": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/copyw -o run "
             "-- python3 $R/bench.py --copy-calibration",
    "sq": "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_WAVES SQ_BUSY_CYCLES "
          "SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS --output-format csv "
          f"-d $R/gpurun_out/prof/sq -o run -- {_BENCH} --steps 5 --warmup 2 --config-reps 5",
    "pipe": "rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_ACTIVE_INST_ANY "
            "SQ_ACTIVE_INST_VALU SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE TA_TA_BUSY_sum TD_TD_BUSY_sum "
            "TCP_TOTAL_CACHE_ACCESSES_sum --output-format csv "
            f"-d $R/gpurun_out/prof/pipe -o run -- {_BENCH} --steps 5 --warmup 2 --config-reps 5",
}


def _kernel_key(name: str, blocks: int) -> str:
    """A kernel instantiation at one launch size: 'fwd_mfma<2, 2, 8, 4, false>|4096'."""
    n = name.split("(")[0].replace("void ", "").replace("dwc::", "").strip()
    return f"{n}|{blocks}"


def _trace_dispatches(d):
    """(kernel key, duration us) of every traced libdwc dispatch, in
    dispatch order (the library's kernels run on one stream)."""
    rows = sorted(_csv_rows(os.path.join(d, "trace"), "*kernel_trace.csv"),
                  key=lambda r: int(r["Start_Timestamp"]))
    out = []
    for r in rows:
        if "dwc::" not in r["Kernel_Name"]:
            continue  # torch's own copies and fills
        blocks = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        out.append((_kernel_key(r["Kernel_Name"], blocks),
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    return out


def case_shape(workload, case):
    """(Shape, dtype) of a per-configuration entry's case key."""
    wl = WORKLOADS[workload]
    for sh in wl["shapes"]:
        for dt in wl["dtypes"]:
            if config_label(workload, sh, dt)[1] == case:
                return sh, dt
    raise KeyError((workload, case))


def _expected_launches(dwc, details):
    """The library calls of the traced run in order, each as (tag, kernel
    specs): the headline step loop, its per-op pass, then every
    configuration group's three passes (3 launches per op, the warm-up,
    the timed launches), as bench.py issues them."""
    seq = []
    s_h = WORKLOADS[HEADLINE]["shapes"][HEADLINE_SHAPE]
    hk = [(op, kernels_of(dwc, s_h, op, HEADLINE_DTYPE)) for op in HEADLINE_OPS]
    for _ in range(PROFILE_WARMUP + PROFILE_STEPS):
        seq += [(None, k) for _, k in hk]
    for op, k in hk:
        seq += [(("head", op), k)] * PROFILE_STEPS
    groups = []
    for i, r in enumerate(details):
        key = (r["workload"], r["case"], r["algo"])
        if not groups or groups[-1][0] != key:
            groups.append((key, []))
        groups[-1][1].append(i)
    for _, idx in groups:
        for phase in ("t1", "warm"):
            for i in idx:
                r = details[i]
                n = {"t1": 3, "warm": r["warm"]}[phase]
                seq += [(None, r["kernels"].split("+"))] * n
        for i in idx:  # per op: a graph replayed twice (the second timed), one eager check
            r = details[i]
            k = r["kernels"].split("+")
            if r.get("timing") == "graph":
                seq += [(None, k)] * r["reps"] + [(("cfg", i), k)] * r["reps"] + [(None, k)]
            else:
                seq += [(("cfg", i), k)] * r["reps"]
    return seq


def _align(dispatches, seq):
    """Per tag, the summed kernel time of each of its launches, walking the
    traced dispatches against the expected launches (names and launch
    sizes must agree)."""
    out, pos = {}, 0
    for tag, specs in seq:
        t = 0.0
        for spec in specs:
            key, us = dispatches[pos]
            if not kernel_matches([key], spec):
                raise RuntimeError(f"trace dispatch {pos} is {key}, expected {spec}")
            t += us
            pos += 1
        if tag is not None:
            out.setdefault(tag, []).append(t)
    if pos != len(dispatches):
        raise RuntimeError(f"{len(dispatches) - pos} traced dispatches left over")
    return out


def summarize_profile(d):
    """Write profiles/<headline>.kernel_trace.md, profiles/configs.kernel_trace.md,
    the HBM traffic summary and traffic.json from the rocprofv3 output of
    this benchmark under d."""
    os.makedirs(PROFILES, exist_ok=True)
    cd = "cd /tmp && export TMPDIR=/tmp && "
    traced = None
    for ln in open(os.path.join(d, "trace.log")):
        if ln.startswith("{") and '"metric"' in ln:
            traced = json.loads(ln)
    details = [json.loads(ln) for ln in open(os.path.join(d, "details.jsonl"))]
    import depthwise_convolution_dwc_amd as dwc
    for r in details:  # the kernels each entry launches, from its plan
        s_r, dt_r = case_shape(r["workload"], r["case"])
        r["kernels"] = "+".join(kernels_of(dwc, s_r, r["op"], dt_r, r["algo"]))
    disp = _trace_dispatches(d)
    per = _align(disp, _expected_launches(dwc, details))
    s_h = WORKLOADS[HEADLINE]["shapes"][HEADLINE_SHAPE]
    # headline step: the per-op pass (PROFILE_STEPS launches of each op back
    # to back) against the JSON line's event times
    names = {}
    for k, _ in disp:
        names.setdefault(k, 0)
        names[k] += 1
    lines = ["| op | kernels (template arguments, workgroups) | rocprofv3 avg us, per-op pass | "
             "JSON line `ops.<op>.ms`, us |", "|---|---|---|---|"]
    for op in HEADLINE_OPS:
        ks = kernels_of(dwc, s_h, op, HEADLINE_DTYPE)
        full = [kernel_matches(names, k)[0] for k in ks]
        js = traced["ops"][op]["ms"] * 1e3 if traced else float("nan")
        lines.append(f"| {op} | {' + '.join('`' + f.replace('|', '`, ') for f in full)} | "
                     f"{np.mean(per[('head', op)]):.2f} | {js:.2f} |")
    trace_md = f"""# Kernel trace: mixed-precision step, N=128 28x28 C=512 31x31 pad 15, fp16 operands

One benchmark step = forward + data gradient + filter gradient on the same
batch (the default `bench.py` workload; fp16 operands, fp32 accumulation and
outputs, the library's kernel choice: the packed-MFMA kernels), on one
MI355X, buffer sets rotating over >= 1 GiB (no Infinity-Cache reuse).  The
traced run launches each op {PROFILE_WARMUP} + {PROFILE_STEPS} times in the
step loop, then {PROFILE_STEPS} times back to back in the per-op pass whose
HIP-event timings give the JSON line's per-op durations (`ops`), and then
every per-configuration entry ({PROFILE_REPS} timed launches each); the
kernel names below carry their template arguments and the workgroup count.

Command (repository root `$R`):

```
{cd}{PROFILE_CMDS["trace"]}
cd $R && python3 bench.py --summarize-profile gpurun_out/prof
```

Durations from the dispatch timestamps of `run_kernel_trace.csv`, each
dispatch matched to the launch bench.py issued (kernel name and workgroup
count checked in order); the last two columns compare the kernels' rocprofv3
average over the per-op pass with the event time the JSON line printed for
that op (under the profiler both run a few percent slower than in an
unprofiled run):

{chr(10).join(lines)}

The data gradient is the forward kernel on dY with the filter turned by
180 degrees (`FLIP` = true); the filter gradient is `wgrad_mfma` followed by
`reduce_partials`.  Template arguments: `fwd_mfma_batch` operand dtype
(2 = fp16), channels per workgroup, FLIP; `fwd_mfma` dtype, 16-tap filter
fragments, channels per workgroup, tiles, FLIP; `wgrad_mfma` dtype, 16-tap
fragments of FW and FH, 32-column chunks, staging items per thread.
"""
    with open(os.path.join(PROFILES, PROFILE_NAME + ".kernel_trace.md"), "w") as f:
        f.write(trace_md)

    # every per-configuration entry: the traced durations of its timed
    # launches beside the bench's event time
    clines = ["| config | case | op | algo | kernels, workgroups | rocprofv3 avg us | event us | "
              "GFLOP/s | fraction |", "|---|---|---|---|---|---|---|---|---|"]
    for i, r in enumerate(details):
        full = [kernel_matches(names, k)[0] for k in r["kernels"].split("+")]
        v = float(np.mean(per[("cfg", i)]))
        clines.append(f"| {r['config']} | {r['case']} | {r['op']} | {r['algo']} | "
                      f"{'; '.join('`' + f.replace('|', '`, ') for f in full)} | {v:.1f} | "
                      f"{r['ms'] * 1e3:.1f} | {r['gflops']:.0f} | {r['roofline_frac']:.3f} |")
    cfg_md = f"""# Kernel trace: every per-configuration entry of the benchmark

The same traced run as `{PROFILE_NAME}.kernel_trace.md` (command there).
Each configuration entry (the five configurations of the target and the
measured "next" rows) is timed alone: {PROFILE_REPS} launches on rotating
buffer sets, captured in a HIP graph that is replayed between two events
after a warm-up (so short kernels are not timed at the rate the host
issues them); "event us" is the bench's HIP-event time per launch of that
entry, "rocprofv3 avg us" the traced durations of
its kernels summed per launch and averaged over its {PROFILE_REPS} timed
launches (each traced dispatch matched in order to the launch bench.py
issued, kernel name and workgroup count checked).  Fraction: of the literal roofline min(8 TB/s x eta_D / operand
bytes, peak), peak 157.3 TFLOP/s (fp32 operands), 2.5 PFLOP/s (bf16/fp16
operands), 5.0 PFLOP/s (fp8 operands).  Template arguments: the operand
dtype first (0 fp32, 1 bf16, 2 fp16, 3 e4m3), also for the fp32
matrix-core kernels (`fwd_mfma_f32<dtype, band width, 4-column tiles per
wave, FLIP>`, `wgrad_mfma_f32<dtype, 4-column filter tiles, 4-column output
groups per wave>`, 16-bit operands widened to fp32 on load), except
`fwd_mfma_f32n<band width, tiles, FLIP>` (fp32 only, 4 images as the
matrix rows).

{chr(10).join(clines)}
"""
    with open(os.path.join(PROFILES, "configs.kernel_trace.md"), "w") as f:
        f.write(cfg_md)

    def per_kernel(sub, counter):
        acc = {}
        for r in _csv_rows(os.path.join(d, sub), "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            blocks = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            acc.setdefault(_kernel_key(r["Kernel_Name"], blocks), []).append(
                float(r["Counter_Value"]) * 1024.0)
        return {k: float(np.mean(v)) for k, v in acc.items()}

    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    cf, cw = per_kernel("copyf", "FETCH_SIZE"), per_kernel("copyw", "WRITE_SIZE")
    copy_bytes = 256 * 1024 * 1024  # the calibration copy moves 256 MiB each way
    ck = [k for k in cf if "copyBuffer" in k]
    ckw = [k for k in cw if "copyBuffer" in k]
    f_scale = copy_bytes / cf[ck[0]] if ck else 1.0
    w_scale = copy_bytes / cw[ckw[0]] if ckw else 1.0
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        fb, wb = fetch.get(k, 0.0) * f_scale, write.get(k, 0.0) * w_scale
        kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    out = {"source_hash": kernel_source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": kernels}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    tl = ["| kernel, workgroups | FETCH bytes/launch | WRITE bytes/launch | total |",
          "|---|---|---|---|"]
    for k, e in kernels.items():
        if any(x in k for x in ("copyBuffer", "elementwise", "fill", "Kernel")):
            continue
        tl.append(f"| `{k.replace('|', '`, ')} | {e['fetch_bytes'] / 1e6:.1f} MB | "
                  f"{e['write_bytes'] / 1e6:.1f} MB | {e['bytes_per_launch'] / 1e6:.1f} MB |")
    cmds = "\n".join(cd + PROFILE_CMDS[k] for k in ("fetch", "write", "copyf", "copyw"))
    hk = [kernels_of(dwc, s_h, op, HEADLINE_DTYPE) for op in HEADLINE_OPS]
    hl = []
    for op, ks in zip(HEADLINE_OPS, hk):
        m = op_model(s_h, op, HEADLINE_DTYPE)
        got = sum(kernels[k]["bytes_per_launch"] for kp in ks for k in kernels if k.startswith(kp)
                  and kernels[k]["bytes_per_launch"] == max(
                      kernels[q]["bytes_per_launch"] for q in kernels if q.startswith(kp)))
        hl.append(f"| {op} | {' + '.join(ks)} | {m['bytes'] / 1e6:.1f} MB | {got / 1e6:.1f} MB | "
                  f"{got / m['bytes']:.3f} |")
    traffic_md = f"""# HBM traffic per launch: every kernel of the benchmark

Per-dispatch `FETCH_SIZE` and `WRITE_SIZE` (KiB, rocprofv3 derived counters,
each in a run of its own), averaged over the launches of each kernel at each
launch size and scaled by what the same counters read for a plain 256 MiB
device copy (`bench.py --copy-calibration`, the runtime's copyBuffer
kernel): on this MI355X `FETCH_SIZE` reads {1 / f_scale:.3f} of the copied
bytes (scale {f_scale:.3f}) and `WRITE_SIZE` {1 / w_scale:.3f} (scale
{w_scale:.3f}).  One calibration serves every kernel; it assumes the
counters see a kernel's requests as they see the copy's (whole 64-byte and
128-byte lines).

Commands (repository root `$R`):

```
{cmds}
cd $R && python3 bench.py --summarize-profile gpurun_out/prof
```

Headline step (N=128 28x28 C=512 31x31 pad 15, fp16 operands): measured
against algorithmic bytes (operands read once, fp32 output written once):

| op | kernels | algorithmic | measured | ratio |
|---|---|---|---|---|
{chr(10).join(hl)}

Every kernel at every launch size of the run:

{chr(10).join(tl)}

The same numbers are in `traffic.json`, which `bench.py` reads for the
`traffic` field of its roofline entry while the kernel sources are unchanged
(their hash is stored with the data).
"""
    with open(os.path.join(PROFILES, PROFILE_NAME + ".hbm_traffic.md"), "w") as f:
        f.write(traffic_md)

    # SQ, memory-pipeline and occupancy figures of every kernel: per-wave
    # instruction mix, matrix-core busy fraction, LDS bank conflicts, the
    # waves' issue and wait fractions, TA/TD busy fractions, L1 accesses per
    # load instruction, and the waves per SIMD its resources allow
    def counters(sub):
        out = {}
        for r in _csv_rows(os.path.join(d, sub), "*counter_collection.csv"):
            if "dwc::" not in r["Kernel_Name"]:
                continue
            blocks = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            key = _kernel_key(r["Kernel_Name"], blocks)
            out.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        return {k: {c: float(np.mean(v)) for c, v in cs.items()} for k, cs in out.items()}
    sq, pipe = counters("sq"), counters("pipe")
    res = {}  # kernel key -> (LDS bytes, workgroup size, workgroups), from the trace
    for r in _csv_rows(os.path.join(d, "trace"), "*kernel_trace.csv"):
        if "dwc::" not in r["Kernel_Name"]:
            continue
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        blocks = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        res[_kernel_key(r["Kernel_Name"], blocks)] = (int(r["LDS_Block_Size"]), wg, blocks)
    # dynamic LDS of the packed kernels: the trace's LDS column shows static
    # LDS only, so take the plan's figure for each launch
    def plan_lds(s_, op, dt_, algo="auto"):
        p_ = dwc.problem(s_.n, s_.h, s_.w, s_.c, s_.fh, s_.fw, (s_.stride_h, s_.stride_w),
                         (s_.pad_h, s_.pad_w), DTYPE_CODE[dt_], algo)
        desc = dwc.plan_describe(p_, {"fwd": 0, "bwd_data": 1, "bwd_filter": 2}[op])
        kv_ = dict(t.split("=", 1) for t in desc.split()[2:] if "=" in t)
        return int(kv_.get("lds", 0))
    for s_, op, dt_, algo, ks_ in (
            [(s_h, op, HEADLINE_DTYPE, "auto", kernels_of(dwc, s_h, op, HEADLINE_DTYPE))
             for op in HEADLINE_OPS] +
            [(case_shape(r["workload"], r["case"])[0], r["op"],
              case_shape(r["workload"], r["case"])[1], r["algo"], r["kernels"].split("+"))
             for r in details]):
        lds_b = plan_lds(s_, op, dt_, algo)
        if lds_b:
            for k in kernel_matches(list(res), ks_[0]):
                res[k] = (max(res[k][0], lds_b),) + res[k][1:]
    # registers: the compiler's resource usage, recorded when the library was
    # built (the trace's register columns are not used: on this device they
    # read half the allocation)
    regs_of = {}
    rpath = os.path.join(ROOT, "depthwise_convolution_dwc_amd", "kernel_resources.json")
    if os.path.exists(rpath):
        for k, v in json.load(open(rpath)).items():
            regs_of[k.replace("dwc::", "")] = v

    def occupancy(key):
        """Waves per SIMD: the lowest of what the registers allow (the
        compiler's figure), the LDS (160 KiB per CU, whole workgroups) and
        what the launch provides (1024 SIMDs)."""
        if key not in res:
            return "-"
        lds_b, wg, blocks = res[key]
        rv = regs_of.get(key.split("|")[0], {})
        wpg = max(1, -(-wg // 64))
        by_regs = rv.get("waves_per_simd", 8)
        by_lds = (163840 // lds_b) * wpg / 4 if lds_b else 8
        by_launch = blocks * wpg / 1024
        regs = rv.get("vgprs", 0) + rv.get("agprs", 0)
        return (f"{min(8, by_regs, by_lds, by_launch):.1f} ({regs or '?'} VGPRs, "
                f"{lds_b / 1024:.0f} KiB)")

    def sq_row(key):
        m = sq.get(key, {})
        w = max(m.get("SQ_WAVES", 1.0), 1.0)
        # SQ_BUSY_CYCLES sums the shader engines (32 on MI355X, 8 CUs each);
        # SQ_VALU_MFMA_BUSY_CYCLES sums the SIMDs (1024)
        busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024 / max(m.get("SQ_BUSY_CYCLES", 0) / 32,
                                                                     1.0)
        conf = m.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(m.get("SQ_ACTIVE_INST_LDS", 1.0), 1.0)
        p = pipe.get(key, {})
        wc = max(p.get("SQ_WAVE_CYCLES", 0.0), 1.0)
        # GRBM_GUI_ACTIVE sums the 8 XCDs; the TA and TD counters the 256 CUs
        kc = max(p.get("GRBM_GUI_ACTIVE", 0.0) / 8, 1.0)
        vm = max(p.get("SQ_INSTS_VMEM_RD", 0.0), 1.0)
        return (f"| `{key.replace('|', '`, ')} | {occupancy(key)} | "
                f"{m.get('SQ_INSTS_VALU', 0) / w:.0f} | {m.get('SQ_INSTS_MFMA', 0) / w:.0f} | "
                f"{m.get('SQ_INSTS_LDS', 0) / w:.0f} | {busy:.2f} | {conf:.2f} | "
                f"{p.get('SQ_ACTIVE_INST_ANY', 0) / wc:.2f} | {p.get('SQ_WAIT_ANY', 0) / wc:.2f} | "
                f"{p.get('TA_TA_BUSY_sum', 0) / 256 / kc:.2f} | "
                f"{p.get('TD_TD_BUSY_sum', 0) / 256 / kc:.2f} | "
                f"{p.get('TCP_TOTAL_CACHE_ACCESSES_sum', 0) / vm:.1f} |")

    sq_head = ["| kernel, workgroups | waves / SIMD | VALU / wave | MFMA / wave | LDS / wave | "
               "matrix cores busy | LDS conflict / LDS active | issuing | waiting | TA busy | "
               "TD busy | L1 accesses / load |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    step_keys = set()
    for op in HEADLINE_OPS:
        for k in kernels_of(dwc, s_h, op, HEADLINE_DTYPE):
            step_keys.update(kernel_matches(list(sq), k))
    sl = sq_head + [sq_row(k) for k in sorted(step_keys)]
    cl = sq_head + [sq_row(k) for k in sorted(sq) if k not in step_keys]
    legend = f"""Columns, each counter averaged over the dispatches of one kernel at one
launch size (rocprofv3 derived counters, two runs of their own):
- waves / SIMD: the lowest of what the kernel's registers allow (the
  compiler's resource usage, recorded in `kernel_resources.json` when the
  library is built), its LDS (160 KiB per CU, whole workgroups; the plan's
  dynamic LDS, else the trace's static figure) and its launch size (1024
  SIMDs);
- VALU, MFMA, LDS: instructions per wave (`SQ_INSTS_*` / `SQ_WAVES`);
- matrix cores busy: `SQ_VALU_MFMA_BUSY_CYCLES` per SIMD over
  `SQ_BUSY_CYCLES` per shader engine;
- LDS conflict / LDS active: `SQ_LDS_BANK_CONFLICT` over
  `SQ_ACTIVE_INST_LDS`;
- issuing, waiting: `SQ_ACTIVE_INST_ANY` and `SQ_WAIT_ANY` over
  `SQ_WAVE_CYCLES` (fractions of the waves' resident time);
- TA busy, TD busy: `TA_TA_BUSY_sum` and `TD_TD_BUSY_sum` per CU over
  `GRBM_GUI_ACTIVE` per XCD (the vector-memory address and data units);
- L1 accesses / load: `TCP_TOTAL_CACHE_ACCESSES_sum` over
  `SQ_INSTS_VMEM_RD`: cache lines a load instruction touches (2 for a
  wave's 256 contiguous bytes, up to 64 for 64 scattered pieces).

Commands (repository root `$R`):

```
{cd}{PROFILE_CMDS["sq"]}
{cd}{PROFILE_CMDS["pipe"]}
cd $R && python3 bench.py --summarize-profile gpurun_out/prof
```
"""
    sq_md = f"""# SQ and memory-pipeline counters: mixed-precision step, N=128 28x28 C=512 31x31 pad 15, fp16 operands

The default benchmark step's kernels (forward, data gradient, filter
gradient and its reduction).  The same figures for every other kernel of
the benchmark's per-configuration entries are in `configs.sq_counters.md`.

{legend}
{chr(10).join(sl)}
"""
    cfg_sq_md = f"""# SQ and memory-pipeline counters: every per-configuration entry's kernels

Every kernel the benchmark's per-configuration entries launch (the five
configurations of the target, the strided backward and fp8 rows), except
the default step's, which are in `{PROFILE_NAME}.sq_counters.md`.  Kernel
names carry their template arguments (operand dtype first: 0 fp32, 1 bf16,
2 fp16, 3 e4m3, 4 e5m2; the fp32 matrix-core kernels take
`fwd_mfma_f32<dtype, band width, 4-column tiles per wave, FLIP>` and
`wgrad_mfma_f32<dtype, 4-column filter tiles, 4-column output groups per
wave>`, their fp32-only images variant `fwd_mfma_f32n<band width, tiles,
FLIP>`)
and the workgroup count, which tells the launch sizes of one kernel apart;
`configs.kernel_trace.md` maps them to the configurations.

{legend}
{chr(10).join(cl)}
"""
    with open(os.path.join(PROFILES, "configs.sq_counters.md"), "w") as f:
        f.write(cfg_sq_md)
    with open(os.path.join(PROFILES, PROFILE_NAME + ".sq_counters.md"), "w") as f:
        f.write(sq_md)
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

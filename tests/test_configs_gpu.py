"""GPU parity at the full sizes of the named workloads, through the same
library calls (and so the same launch configuration) the benchmark times.
Every element of every output is compared with the float64 oracle over the
whole tensor: relative L2 error per tensor and an elementwise bound against
the same operation on |operands|.  Half-precision and fp8 workloads run both
the library's choice (the packed-MFMA kernels where they apply) and the
vector kernels, which the benchmark times side by side."""

import functools

import numpy as np
import pytest

import oracle
from dwc_inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import check_parity, dwc, log, sync, to_device  # noqa: E402


def _cases():
    for name, wl in WORKLOADS.items():
        for s in wl["shapes"]:
            for dt in wl["dtypes"]:
                for op in wl["ops"]:
                    yield name, s, dt, op


ALL_CASES = list(_cases())


def _id(c):
    name, s, dt, op = c
    return f"{name}-{s.h}x{s.w}c{s.c}k{s.fh}s{s.stride_h}-{dt}-{op}"


def _vals(op):
    """Operand values for the oracle: fp8 codes through the oracle's own
    decoder, other dtypes as generated (exact in float32)."""
    if op.dtype in oracle.FP8_FORMATS:
        return oracle.fp8_decode(op.stored, op.dtype)
    return op.values


@functools.lru_cache(maxsize=1)
def _inputs(name, s, dt):
    """Seeded inputs of one workload shape, on the host and on the device
    (kept for the three operations of the same case)."""
    wl = WORKLOADS[name]
    inp = make_inputs(s, dt, seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
    return inp, to_device(inp.x), to_device(inp.w), to_device(inp.dy)


def _oracle(op, s, inp):
    """The whole output tensor, and the same operation on |operands|."""
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        a, b = _vals(inp.x), _vals(inp.w)
        f = lambda u, v: oracle.fwd(u, v, stride, pad)
    elif op == "bwd_data":
        a, b = _vals(inp.dy), _vals(inp.w)
        f = lambda u, v: oracle.bwd_data(u, v, (s.h, s.w), stride, pad)
    else:
        a, b = _vals(inp.x), _vals(inp.dy)
        f = lambda u, v: oracle.bwd_filter(u, v, (s.fh, s.fw), stride, pad)
    return f(a, b), f(np.abs(a), np.abs(b))


@pytest.mark.parametrize("case", ALL_CASES, ids=_id)
def test_workload_parity(case):
    name, s, dt, op = case
    log(f"case {name} {s} {dt} {op}")
    inp, x, w, dy = _inputs(name, s, dt)
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    algos = ["auto"] if dt == "f32" else ["auto", "direct"]
    got = {}
    for algo in algos:
        if op == "fwd":
            got[algo] = dwc.fwd(x, w, stride, pad, algo=algo)
        elif op == "bwd_data":
            got[algo] = dwc.bwd_data(dy, w, (s.h, s.w), stride, pad, algo=algo)
        else:
            got[algo] = dwc.bwd_filter(x, dy, (s.fh, s.fw), stride, pad, algo=algo)
    sync()
    got = {a: g.double().cpu().numpy() for a, g in got.items()}
    want, mag = _oracle(op, s, inp)
    for algo, g in got.items():
        err, worst = check_parity(g, want, mag, op, s, dt, what=f"{op} {algo}")
        log(f"  {algo}: rel_l2 = {err:.3e}, worst elementwise error = {worst:.3e} of the bound")

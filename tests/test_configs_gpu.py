"""GPU parity at the full sizes of the named workloads, through the same
library calls (and so the same launch configuration) the benchmark times.
The oracle computes sampled outputs one by one; the small workload is
checked in full."""

import numpy as np
import pytest

import oracle
from dwc_inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import TOL, dwc, gather, log, rel_l2, sample_index, sync, to_device  # noqa: E402


def _cases(name):
    wl = WORKLOADS[name]
    for s in wl["shapes"]:
        for dt in wl["dtypes"]:
            yield name, s, dt


ALL_CASES = [c for name in WORKLOADS for c in _cases(name)]


def _id(c):
    name, s, dt = c
    return f"{name}-{s.h}x{s.w}c{s.c}k{s.fh}s{s.stride_h}-{dt}"


def _check_sampled(op, s, inp, got, k, rng):
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        idx = sample_index(s.y_shape(), k, rng)
        want = oracle.fwd_at(inp.x.values, inp.w.values, idx, stride, pad)
    elif op == "bwd_data":
        idx = sample_index(s.x_shape(), k, rng)
        want = oracle.bwd_data_at(inp.dy.values, inp.w.values, (s.h, s.w), idx, stride, pad)
    else:
        idx = sample_index(s.w_shape(), k, rng)
        want = oracle.bwd_filter_at(inp.x.values, inp.dy.values, (s.fh, s.fw), idx, stride, pad)
    return rel_l2(gather(got, idx), want)


@pytest.mark.parametrize("case", ALL_CASES, ids=_id)
def test_workload_parity(case):
    name, s, dt = case
    wl = WORKLOADS[name]
    small = s.n * s.h * s.w * s.c <= 1 << 16
    inp = make_inputs(s, dt, seed=0, x_dist=wl["x_dist"], w_dist=wl["w_dist"])
    x, w = to_device(inp.x), to_device(inp.w)
    dy = to_device(inp.dy)
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    rng = np.random.default_rng(1)
    big_filter = s.fh * s.fw >= 169
    for op in wl["ops"]:
        log(f"case {name} {s} {dt} {op}")
        if op == "fwd":
            got = dwc.fwd(x, w, stride, pad)
        elif op == "bwd_data":
            got = dwc.bwd_data(dy, w, (s.h, s.w), stride, pad)
        else:
            got = dwc.bwd_filter(x, dy, (s.fh, s.fw), stride, pad)
        sync()
        assert torch.isfinite(got).all().item()
        if small:
            want = {"fwd": lambda: oracle.fwd(inp.x.values, inp.w.values, stride, pad),
                    "bwd_data": lambda: oracle.bwd_data(inp.dy.values, inp.w.values,
                                                        (s.h, s.w), stride, pad),
                    "bwd_filter": lambda: oracle.bwd_filter(inp.x.values, inp.dy.values,
                                                            (s.fh, s.fw), stride, pad)}[op]()
            err = rel_l2(got.double().cpu().numpy(), want)
        else:
            k = {"fwd": 1024, "bwd_data": 1024, "bwd_filter": 48 if big_filter else 128}[op]
            if name == "sweep_n64_stages":
                k = k // 4
            err = _check_sampled(op, s, inp, got, k, rng)
        log(f"  rel_l2 = {err:.3e}")
        assert err <= TOL[dt], (op, err)

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

from gpu_helpers import FP8_EL_TOL, TOL, dwc, gather, log, rel_l2, sample_index, sync, to_device  # noqa: E402


def _cases(name):
    wl = WORKLOADS[name]
    for s in wl["shapes"]:
        for dt in wl["dtypes"]:
            yield name, s, dt


ALL_CASES = [c for name in WORKLOADS for c in _cases(name)]


def _id(c):
    name, s, dt = c
    return f"{name}-{s.h}x{s.w}c{s.c}k{s.fh}s{s.stride_h}-{dt}"


def _vals(op):
    """Operand values for the oracle: fp8 codes through the oracle's own
    decoder, other dtypes as generated (exact in float32)."""
    if op.dtype in oracle.FP8_FORMATS:
        return oracle.fp8_decode(op.stored, op.dtype)
    return op.values


def _check_sampled(op, s, inp, got, k, rng):
    """Relative L2 error over k sampled outputs; for fp8 operands also the
    elementwise bound against the same outputs on |operands|."""
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        idx = sample_index(s.y_shape(), k, rng)
        a, b = _vals(inp.x), _vals(inp.w)
        f = lambda u, v: oracle.fwd_at(u, v, idx, stride, pad)
    elif op == "bwd_data":
        idx = sample_index(s.x_shape(), k, rng)
        a, b = _vals(inp.dy), _vals(inp.w)
        f = lambda u, v: oracle.bwd_data_at(u, v, (s.h, s.w), idx, stride, pad)
    else:
        idx = sample_index(s.w_shape(), k, rng)
        a, b = _vals(inp.x), _vals(inp.dy)
        f = lambda u, v: oracle.bwd_filter_at(u, v, (s.fh, s.fw), idx, stride, pad)
    g, want = gather(got, idx), f(a, b)
    if inp.dtype in oracle.FP8_FORMATS:
        mag = f(np.abs(a), np.abs(b))
        assert np.all(np.abs(g - want) <= FP8_EL_TOL * mag + 1e-30), op
    return rel_l2(g, want)


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
            want = {"fwd": lambda: oracle.fwd(_vals(inp.x), _vals(inp.w), stride, pad),
                    "bwd_data": lambda: oracle.bwd_data(_vals(inp.dy), _vals(inp.w),
                                                        (s.h, s.w), stride, pad),
                    "bwd_filter": lambda: oracle.bwd_filter(_vals(inp.x), _vals(inp.dy),
                                                            (s.fh, s.fw), stride, pad)}[op]()
            err = rel_l2(got.double().cpu().numpy(), want)
        else:
            k = {"fwd": 1024, "bwd_data": 1024, "bwd_filter": 48 if big_filter else 128}[op]
            if name == "sweep_n64_stages":
                k = k // 4
            err = _check_sampled(op, s, inp, got, k, rng)
        log(f"  rel_l2 = {err:.3e}")
        assert err <= TOL[dt], (op, err)

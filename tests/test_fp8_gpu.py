"""GPU parity for fp8 operands (Flash-DWC, TACO, §7, low-bit data types:
operands stored and multiplied in 8 bits, sums in fp32), element by element.

Every kernel family that accepts the problem is compared with the float64
oracle on the decoded codes, by relative L2 error and elementwise against
the same operation on |operands| (the sum of product magnitudes behind each
output), which bounds what a correct fp32-output sum may lose."""

import numpy as np
import pytest

import oracle
from dwc_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import FP8_EL_TOL, TOL, dwc, log, rel_l2, sync, to_device  # noqa: E402

DT = {"e4m3": dwc.FP8_E4M3, "e5m2": dwc.FP8_E5M2}
OPS = {"fwd": 0, "bwd_data": 1, "bwd_filter": 2}

# (n, h, w, c, fh, fw, stride, pad): the sweep (3x3 .. 9x9), register-window
# (other sizes, stride 2), generic and phase (strided data gradient) kernels,
# and the packed-MFMA shapes (C a multiple of 16, widths up to 64)
SHAPES = [
    (2, 14, 14, 64, 7, 7, 1, 3),
    (2, 17, 13, 96, 3, 3, 1, 1),
    (1, 9, 23, 33, 5, 5, 1, 2),
    (2, 20, 20, 64, 7, 7, 2, 3),
    (1, 11, 13, 40, 3, 3, 3, 1),
    (2, 10, 11, 64, 13, 13, 1, 6),
    (2, 28, 28, 64, 13, 13, 1, 6),
    (1, 28, 28, 32, 31, 31, 1, 15),
    (1, 40, 50, 48, 17, 17, 1, 8),
    (2, 9, 64, 16, 5, 9, 1, (2, 4)),
]


def _shape(t):
    n, h, w, c, fh, fw, s, p = t
    sh, sw = (s, s) if isinstance(s, int) else s
    ph, pw = (p, p) if isinstance(p, int) else p
    return Shape(n, h, w, c, fh, fw, sh, sw, ph, pw)


def _oracle(op, s, a, b):
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        return oracle.fwd(a, b, stride, pad)
    if op == "bwd_data":
        return oracle.bwd_data(a, b, (s.h, s.w), stride, pad)
    return oracle.bwd_filter(a, b, (s.fh, s.fw), stride, pad)


def _operands(op, inp):
    if op == "fwd":
        return inp.x, inp.w
    if op == "bwd_data":
        return inp.dy, inp.w
    return inp.x, inp.dy


def _run(op, s, inp, algo):
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        got = dwc.fwd(to_device(inp.x), to_device(inp.w), stride, pad, algo=algo)
    elif op == "bwd_data":
        got = dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (s.h, s.w), stride, pad,
                           algo=algo)
    else:
        got = dwc.bwd_filter(to_device(inp.x), to_device(inp.dy), (s.fh, s.fw), stride, pad,
                             algo=algo)
    sync()
    return got.double().cpu().numpy()


def _algos(op, s, dtype):
    out = []
    for algo in ("auto", "direct", "mfma", "generic"):
        p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                        (s.pad_h, s.pad_w), dtype=DT[dtype], algo=algo)
        if dwc.check(p, OPS[op]) == 0:
            out.append(algo)
    return out


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda t: "x".join(map(str, t[:6])) + f"_s{t[6]}_p{t[7]}")
def test_fp8_parity(shape, op, dtype):
    s = _shape(shape)
    inp = make_inputs(s, dtype, seed=3 + sum(shape[:6]))
    a, b = _operands(op, inp)
    va, vb = oracle.fp8_decode(a.stored, dtype), oracle.fp8_decode(b.stored, dtype)
    want = _oracle(op, s, va, vb)
    mag = _oracle(op, s, np.abs(va), np.abs(vb))
    algos = _algos(op, s, dtype)
    assert "auto" in algos
    for algo in algos:
        log(f"case {shape} {op} {dtype} {algo}")
        got = _run(op, s, inp, algo)
        assert got.shape == want.shape
        assert np.all(np.isfinite(got))
        err = rel_l2(got, want)
        assert err <= TOL[dtype], (algo, err)
        bad = np.abs(got - want) > FP8_EL_TOL * mag + 1e-30
        assert not np.any(bad), (algo, int(bad.sum()), np.argwhere(bad)[:3])


# The 16-image batch-packed kernel with fp8 operands (v_mfma_f32_16x16x32
# fp8 / bf8; C % 16 == 0, N >= 8, input and output widths up to 32), forced
# for every filter height: ragged image groups and row chunks, channel-block
# counts that are not a multiple of the neighbour group, one and two 16-column
# output groups, FH != FW, the widest input, wide padding.
BATCH16_SHAPES = [
    (16, 28, 28, 16, 31, 31, 1, 15),
    (25, 14, 13, 48, 5, 5, 1, 2),
    (9, 30, 32, 64, 17, 17, 1, 8),
    (12, 10, 17, 16, 3, 31, 1, (1, 15)),
    (8, 16, 16, 32, 9, 9, 1, 4),
    (19, 9, 12, 80, 21, 11, 1, (10, 3)),
]


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data"])
@pytest.mark.parametrize("shape", BATCH16_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_p{t[7]}")
def test_fp8_batch16_parity(shape, op, dtype, monkeypatch):
    monkeypatch.setenv("DWC_MFMA_BATCH", "1")
    s = _shape(shape)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT[dtype],
                    algo="mfma")
    d = dwc.plan_describe(p, OPS[op])
    assert " batch=1 " in d and " imgs=16 " in d, d
    inp = make_inputs(s, dtype, seed=11 + sum(shape[:6]))
    a, b = _operands(op, inp)
    va, vb = oracle.fp8_decode(a.stored, dtype), oracle.fp8_decode(b.stored, dtype)
    want = _oracle(op, s, va, vb)
    mag = _oracle(op, s, np.abs(va), np.abs(vb))
    for algo in ("auto", "mfma"):
        log(f"case fp8 batch16 {shape} {op} {dtype} {algo}")
        got = _run(op, s, inp, algo)
        assert np.all(np.isfinite(got))
        err = rel_l2(got, want)
        assert err <= TOL[dtype], (algo, err)
        bad = np.abs(got - want) > FP8_EL_TOL * mag + 1e-30
        assert not np.any(bad), (algo, int(bad.sum()), np.argwhere(bad)[:3])

"""GPU parity at small sizes: every element of the HIP result against the
float64 oracle, for all three operations, all operand dtypes and both kernel
families, over shapes that span several tiles, ragged tails and the
degenerate cases (C not a multiple of 64, filters larger than the image,
stride 2, N = 0, 1x1 filters, widths without a register-window kernel)."""

import numpy as np
import pytest

import oracle
from dwc_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import TOL, check_parity, dwc, el_bound, log, rel_l2, sync, to_device  # noqa: E402

# (n, h, w, c, fh, fw, stride, pad)
SHAPES = [
    (2, 14, 14, 32, 7, 7, 1, 3),
    (2, 17, 13, 96, 3, 3, 1, 1),
    (1, 9, 23, 33, 5, 5, 1, 2),
    (3, 12, 12, 3, 9, 9, 1, 4),
    (2, 10, 11, 64, 13, 13, 1, 6),
    (1, 6, 7, 130, 31, 31, 1, 15),
    (2, 20, 20, 64, 7, 7, 2, 3),
    (1, 5, 40, 70, 3, 5, 1, (1, 2)),
    (1, 7, 7, 1, 31, 31, 1, 15),
    (2, 30, 5, 64, 17, 3, 2, (8, 1)),
    (1, 8, 8, 16, 4, 4, 1, 2),
    (1, 16, 16, 64, 21, 21, 1, 10),
    (1, 16, 19, 64, 27, 27, 1, 13),
    (2, 9, 9, 8, 1, 1, 1, 0),
    (1, 11, 13, 40, 3, 3, 3, 1),
    (1, 33, 35, 128, 7, 7, 1, 0),
    (2, 12, 29, 64, 5, 5, (2, 1), 2),
    # square stride-1 filters with unequal row / column padding (the sweep
    # kernels pad rows and columns separately)
    (2, 13, 17, 64, 3, 3, 1, (1, 0)),
    (1, 12, 15, 96, 5, 5, 1, (0, 2)),
    (2, 11, 20, 64, 7, 7, 1, (3, 1)),
    (1, 16, 13, 128, 9, 9, 1, (2, 4)),
    # padding beyond F-1: the stride-1 data gradient is a forward map with a
    # negative (cropping) padding F-1-pad
    (1, 10, 10, 16, 3, 3, 1, 4),
    (2, 12, 12, 64, 13, 13, 1, 14),
    # widths between the instantiated direct widths: the next wider body
    # with its extra taps skipped (11 on 13, 2 on 3, 15 on 17, 29 on 31,
    # 19 on 21), at stride 1 (all three operations) and 2
    (2, 13, 15, 64, 11, 11, 1, 5),
    (2, 9, 21, 24, 3, 2, 1, (1, 0)),
    (1, 12, 18, 40, 6, 15, 2, (2, 7)),
    (1, 10, 40, 70, 5, 29, 1, (2, 14)),
    (1, 6, 30, 16, 1, 19, 1, (0, 9)),
]


def _shape(t):
    n, h, w, c, fh, fw, s, p = t
    sh, sw = (s, s) if isinstance(s, int) else s
    ph, pw = (p, p) if isinstance(p, int) else p
    return Shape(n, h, w, c, fh, fw, sh, sw, ph, pw)


def _run(op, s: Shape, inp, algo, wgrad_split=0):
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        got = dwc.fwd(to_device(inp.x), to_device(inp.w), stride, pad, algo=algo)
    elif op == "bwd_data":
        got = dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (s.h, s.w), stride, pad,
                           algo=algo)
    else:
        got = dwc.bwd_filter(to_device(inp.x), to_device(inp.dy), (s.fh, s.fw), stride, pad,
                             algo=algo, wgrad_split=wgrad_split)
    sync()
    return got.double().cpu().numpy()


OPS = {"fwd": 0, "bwd_data": 1, "bwd_filter": 2}
DT = {"f32": dwc.F32, "bf16": dwc.BF16, "f16": dwc.F16, "e4m3": dwc.FP8_E4M3,
      "e5m2": dwc.FP8_E5M2}


def _vals(op):
    """Operand values for the oracle: fp8 codes through the oracle's own
    decoder, other dtypes as generated (exact in float32)."""
    if op.dtype in oracle.FP8_FORMATS:
        return oracle.fp8_decode(op.stored, op.dtype)
    return op.values


def _algos(op, s: Shape, dtype):
    """Every kernel family that accepts this problem."""
    out = []
    for algo in ("auto", "direct", "mfma", "generic"):
        p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                        (s.pad_h, s.pad_w), dtype=DT[dtype], algo=algo)
        if dwc.check(p, OPS[op]) == 0:
            out.append(algo)
    return out


def _oracle_op(op, s: Shape):
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    if op == "fwd":
        return lambda a, b: oracle.fwd(a, b, stride, pad)
    if op == "bwd_data":
        return lambda a, b: oracle.bwd_data(a, b, (s.h, s.w), stride, pad)
    return lambda a, b: oracle.bwd_filter(a, b, (s.fh, s.fw), stride, pad)


def _operands(op, inp):
    if op == "fwd":
        return _vals(inp.x), _vals(inp.w)
    if op == "bwd_data":
        return _vals(inp.dy), _vals(inp.w)
    return _vals(inp.x), _vals(inp.dy)


def _want(op, s: Shape, inp):
    return _oracle_op(op, s)(*_operands(op, inp))


def _want_mag(op, s: Shape, inp):
    """The oracle's result and the same operation on |operands| (the scale
    of the elementwise bound)."""
    f, (a, b) = _oracle_op(op, s), _operands(op, inp)
    return f(a, b), f(np.abs(a), np.abs(b))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "e4m3", "e5m2"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda t: "x".join(map(str, t[:6])) + f"_s{t[6]}_p{t[7]}")
def test_small_parity(shape, op, dtype):
    s = _shape(shape)
    inp = make_inputs(s, dtype, seed=sum(shape[:6]))
    want, mag = _want_mag(op, s, inp)
    for algo in _algos(op, s, dtype):
        log(f"case {shape} {op} {dtype} {algo}")
        got = _run(op, s, inp, algo)
        check_parity(got, want, mag, op, s, dtype, what=algo)


@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
def test_empty_batch(op):
    s = Shape(0, 8, 8, 16, 3, 3, 1, 1, 1, 1)
    x = torch.zeros((0, 8, 8, 16), device="cuda")
    w = torch.randn((3, 3, 16), device="cuda")
    if op == "fwd":
        assert dwc.fwd(x, w, 1, 1).shape == (0, 8, 8, 16)
    elif op == "bwd_data":
        assert dwc.bwd_data(x, w, (8, 8), 1, 1).shape == (0, 8, 8, 16)
    else:
        dw = torch.full((3, 3, 16), 7.0, device="cuda")
        dwc.bwd_filter(x, x, (3, 3), 1, 1, out=dw)
        sync()
        assert torch.count_nonzero(dw).item() == 0
    del s


@pytest.mark.parametrize("split", [1, 2, 5, 24])
def test_wgrad_split_invariance(split):
    s = Shape(3, 8, 12, 80, 5, 5, 1, 1, 2, 2)
    inp = make_inputs(s, "f32", seed=12)
    want, mag = _want_mag("bwd_filter", s, inp)
    got = _run("bwd_filter", s, inp, "auto", wgrad_split=split)
    check_parity(got, want, mag, "bwd_filter", s, "f32")


@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
def test_run_to_run_bitwise(op):
    s = Shape(4, 24, 24, 128, 13, 13, 1, 1, 6, 6)
    inp = make_inputs(s, "f32", seed=5)
    a = _run(op, s, inp, "auto")
    b = _run(op, s, inp, "auto")
    np.testing.assert_array_equal(a, b)


def test_outputs_fully_overwritten():
    """Outputs start as NaN; every element must be written."""
    s = Shape(2, 13, 11, 70, 7, 7, 1, 1, 3, 3)
    inp = make_inputs(s, "f32", seed=8)
    y = torch.full(s.y_shape(), float("nan"), device="cuda")
    dwc.fwd(to_device(inp.x), to_device(inp.w), 1, 3, out=y)
    dx = torch.full(s.x_shape(), float("nan"), device="cuda")
    dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (13, 11), 1, 3, out=dx)
    dw = torch.full(s.w_shape(), float("nan"), device="cuda")
    dwc.bwd_filter(to_device(inp.x), to_device(inp.dy), (7, 7), 1, 3, out=dw)
    sync()
    for t in (y, dx, dw):
        assert torch.isfinite(t).all().item()


def test_caller_stream_is_used():
    s = Shape(2, 20, 20, 64, 7, 7, 1, 1, 3, 3)
    inp = make_inputs(s, "f32", seed=9)
    st = torch.cuda.Stream()
    x, w = to_device(inp.x), to_device(inp.w)
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(st):
        y = dwc.fwd(x, w, 1, 3)
    st.synchronize()
    assert rel_l2(y.double().cpu().numpy(), _want("fwd", s, inp)) <= 1e-5


# Shapes for the packed-MFMA kernel (bf16/fp16, stride 1): every tile shape
# (column groups per tile 1, 2, 4; one or two tiles), both fragment counts,
# a half-filled channel block, FH != FW, no padding, and data-gradient
# padding larger than F-1 (a cropping forward map); for the filter gradient
# every fragment count (16-tap slices of FW and FH, 32-column chunks of W)
# and one or two staging items per thread.
MFMA_SHAPES = [
    (1, 6, 6, 16, 3, 3, 1, 1),
    (2, 20, 13, 24, 5, 5, 1, 2),
    (1, 28, 28, 32, 13, 13, 1, 6),
    (1, 9, 40, 16, 7, 5, 1, 3),
    (1, 11, 11, 8, 31, 31, 1, 15),
    (2, 19, 21, 40, 17, 17, 1, 8),
    (1, 12, 12, 16, 32, 32, 1, 16),
    (2, 7, 7, 16, 3, 3, 1, 0),
    (1, 10, 10, 16, 3, 3, 1, 4),
    (1, 30, 64, 16, 9, 1, 1, (4, 0)),
    (3, 16, 16, 8, 1, 31, 1, (0, 15)),
    (2, 36, 32, 8, 3, 3, 1, 1),
    (1, 22, 64, 8, 5, 3, 1, (2, 1)),
    (2, 12, 50, 8, 20, 20, 1, (9, 10)),
    (1, 20, 60, 8, 17, 17, 1, 8),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
@pytest.mark.parametrize("shape", MFMA_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_p{t[7]}")
def test_mfma_parity(shape, op, dtype):
    s = _shape(shape)
    assert "mfma" in _algos(op, s, dtype), "shape meant for the packed-MFMA kernel"
    inp = make_inputs(s, dtype, seed=31 + sum(shape[:6]))
    want, mag = _want_mag(op, s, inp)
    log(f"case mfma {shape} {op} {dtype}")
    got = _run(op, s, inp, "mfma")
    check_parity(got, want, mag, op, s, dtype, what="mfma")


def _misaligned(t):
    """A copy of t whose storage starts 2 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def test_mfma_misaligned_tensors():
    """AUTO falls back to the vector kernels; forcing MFMA is an error."""
    s = Shape(2, 14, 14, 32, 7, 7, 1, 1, 3, 3)
    inp = make_inputs(s, "bf16", seed=3)
    want = _want("fwd", s, inp)
    x = _misaligned(to_device(inp.x))
    w = to_device(inp.w)
    got = dwc.fwd(x, w, 1, 3)
    sync()
    assert rel_l2(got.double().cpu().numpy(), want) <= TOL["bf16"]
    with pytest.raises(dwc.DwcError):
        dwc.fwd(x, w, 1, 3, algo="mfma")


@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
def test_mfma_outputs_fully_overwritten(op):
    s = Shape(2, 21, 19, 40, 9, 9, 1, 1, 4, 4)
    inp = make_inputs(s, "bf16", seed=4)
    if op == "fwd":
        y = torch.full(s.y_shape(), float("nan"), device="cuda")
        dwc.fwd(to_device(inp.x), to_device(inp.w), 1, 4, out=y, algo="mfma")
    elif op == "bwd_filter":
        # NaN in dW and in every workspace byte: each partial is written
        # before the reduction reads it
        y = torch.full((9, 9, 40), float("nan"), device="cuda")
        p = dwc.problem(2, 21, 19, 40, 9, 9, 1, 4, dtype=dwc.BF16, algo="mfma")
        ws = torch.full((dwc.workspace_size(p) // 4,), float("nan"), device="cuda")
        dwc.bwd_filter(to_device(inp.x), to_device(inp.dy), (9, 9), 1, 4, out=y,
                       workspace=ws, algo="mfma")
    else:
        y = torch.full(s.x_shape(), float("nan"), device="cuda")
        dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (21, 19), 1, 4, out=y, algo="mfma")
    sync()
    want, mag = _want_mag(op, s, inp)
    check_parity(y.double().cpu().numpy(), want, mag, op, s, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
def test_mfma_many_workgroups(dtype, op):
    """Several row chunks and channel blocks per image: every workgroup
    stages its own rows and filter fragments."""
    s = _shape((3, 40, 20, 48, 7, 7, 1, 3))
    assert "mfma" in _algos(op, s, dtype)
    inp = make_inputs(s, dtype, seed=40)
    got = _run(op, s, inp, "mfma")
    want, mag = _want_mag(op, s, inp)
    check_parity(got, want, mag, op, s, dtype)


@pytest.mark.parametrize("split", [1, 2, 3, 5])
def test_mfma_wgrad_batch_slices(split):
    """Slices of several images each (split < N): every slice accumulates
    its images in registers, the reduction sums the slices in a fixed order,
    so the result is run-to-run bitwise identical."""
    s = _shape((5, 13, 17, 24, 7, 5, 1, (3, 2)))
    inp = make_inputs(s, "bf16", seed=50 + split)
    want, mag = _want_mag("bwd_filter", s, inp)
    log(f"case mfma wgrad split={split}")
    got = _run("bwd_filter", s, inp, "mfma", wgrad_split=split)
    check_parity(got, want, mag, "bwd_filter", s, "bf16")
    again = _run("bwd_filter", s, inp, "mfma", wgrad_split=split)
    assert np.array_equal(got, again)


@pytest.mark.parametrize("rows", [1, 2, 3, 6, 7, 11])
@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
@pytest.mark.parametrize("shape", [(2, 23, 21, 64, 7, 7, 1, 3), (2, 17, 19, 64, 3, 3, 1, 1),
                                   (1, 20, 14, 128, 5, 5, 1, (2, 1)), (1, 19, 16, 64, 9, 9, 1, 4)],
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_p{t[7]}")
def test_sweep_row_chunks(shape, op, rows, monkeypatch):
    """The sweep kernels cut each image into chunks of R output rows that
    re-read F-1 halo rows and skip the products that fall outside the
    chunk or the image: every chunk size, including R < F and ragged last
    chunks, matches the oracle."""
    monkeypatch.setenv("DWC_SWEEP_ROWS", str(rows))
    s = _shape(shape)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), algo="direct")
    d = dwc.plan_describe(p, OPS[op])
    assert " sweep " in d and f" rows={rows} " in d, d
    inp = make_inputs(s, "f32", seed=60 + rows)
    log(f"case sweep rows={rows} {shape} {op}")
    got = _run(op, s, inp, "direct")
    want, mag = _want_mag(op, s, inp)
    check_parity(got, want, mag, op, s, "f32")


# Strided data gradient (the phase kernel): strides 2 and 3, square and
# non-square filters, even filters, sub-filters that need chunking (KM > 8),
# padding larger than the stride, dims that are not multiples of the stride,
# ragged channel blocks and a stride larger than the filter.
STRIDED_DGRAD_SHAPES = [
    (2, 9, 10, 64, 3, 3, 2, 1),
    (1, 11, 13, 70, 31, 31, 2, 15),
    (1, 10, 10, 64, 5, 5, 3, 2),
    (2, 8, 8, 64, 1, 1, 2, 0),
    (1, 9, 9, 64, 4, 6, 2, (1, 2)),
    (2, 17, 16, 96, 7, 7, 2, 3),
    (1, 12, 15, 130, 9, 9, 2, 4),
    (1, 20, 9, 64, 17, 5, 2, (8, 2)),
    (1, 7, 7, 33, 3, 3, 3, 0),
    (1, 13, 11, 64, 21, 21, 2, 10),
    (1, 6, 6, 64, 2, 2, 2, 0),
    (2, 28, 28, 128, 7, 7, 2, 3),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", STRIDED_DGRAD_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_s{t[6]}_p{t[7]}")
def test_strided_dgrad_phase(shape, dtype):
    s = _shape(shape)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                    (s.pad_h, s.pad_w), dtype=DT[dtype])
    assert " phase " in dwc.plan_describe(p, 1)
    inp = make_inputs(s, dtype, seed=70 + sum(shape[:6]))
    want, mag = _want_mag("bwd_data", s, inp)
    log(f"case phase {shape} {dtype}")
    for algo in ("auto", "direct"):
        got = _run("bwd_data", s, inp, algo)
        check_parity(got, want, mag, "bwd_data", s, dtype, what=algo)


def test_strided_dgrad_overwrites_output():
    s = _shape((2, 17, 16, 96, 7, 7, 2, 3))
    inp = make_inputs(s, "f32", seed=5)
    dx = torch.full(s.x_shape(), float("nan"), device="cuda")
    dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (17, 16), 2, 3, out=dx)
    sync()
    want, mag = _want_mag("bwd_data", s, inp)
    check_parity(dx.double().cpu().numpy(), want, mag, "bwd_data", s, "f32")


# Non-finite operands on the vector kernels: IEEE arithmetic, as in the
# oracle.  One +inf and one -inf element (two rows apart, same channel) in
# the input the operation reads pixel by pixel (X for the forward and the
# filter gradient, dY for the data gradient): outputs whose sums take one of
# them are +-inf, those that take both (with products of opposite signs) are
# NaN, and every other output is unaffected.  The packed-MFMA kernels are
# not covered: their Toeplitz band multiplies each staged element by
# structural zeros too, so a non-finite operand turns nearby outputs into NaN
# there; the header states that those kernels need finite operands.
NONFINITE_SHAPES = [
    (2, 14, 14, 64, 7, 7, 1, 3),       # sweep kernels
    (2, 16, 15, 64, 13, 13, 1, 6),     # register-window kernels
    (2, 12, 13, 40, 5, 3, 1, (2, 1)),  # register-window, non-square
    (2, 15, 15, 64, 7, 7, 2, 3),       # stride 2: phase data gradient
    (1, 11, 13, 40, 3, 3, 3, 1),       # stride 3: generic kernels
    (2, 14, 16, 40, 5, 11, 1, (2, 5)), # width 11 on the 13-wide body
    (2, 15, 15, 64, 4, 6, 2, (1, 2)),  # width 6 on the 7-wide body, stride 2
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data", "bwd_filter"])
@pytest.mark.parametrize("shape", NONFINITE_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_s{t[6]}")
def test_nonfinite_operands_vector_kernels(shape, op, dtype):
    s = _shape(shape)
    inp = make_inputs(s, dtype, seed=80 + sum(shape[:6]))
    src = inp.dy if op == "bwd_data" else inp.x
    nn, h = src.values.shape[:2]
    for row, val in ((h // 2 - 1, np.inf), (h // 2 + 1, -np.inf)):
        idx = (nn - 1, row, src.values.shape[2] // 2, 3)
        src.values[idx] = val
        if dtype == "bf16":
            src.stored[idx] = 0x7F80 if val > 0 else 0xFF80
        else:
            src.stored[idx] = val
    want, mag = _want_mag(op, s, inp)
    assert (~np.isfinite(want)).any() and np.isfinite(want).any()
    algos = ["direct", "generic"]
    # AUTO too where it takes a vector kernel (fp32 only: 16-bit AUTO takes
    # the matrix cores at stride 1)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, (s.stride_h, s.stride_w),
                    (s.pad_h, s.pad_w), dtype=DT[dtype])
    if dtype == "f32" and " mfma " not in dwc.plan_describe(p, OPS[op]):
        algos.append("auto")
    for algo in [a for a in _algos(op, s, dtype) if a in algos]:
        log(f"case nonfinite {shape} {op} {dtype} {algo}")
        got = _run(op, s, inp, algo)
        for cls in (np.isnan, np.isposinf, np.isneginf):
            bad = cls(got) != cls(want)
            assert not bad.any(), (algo, cls.__name__, np.argwhere(bad)[:4].tolist())
        fin = np.isfinite(want)
        d = np.abs(got[fin] - want[fin])
        assert np.all(d <= el_bound(op, s, dtype) * mag[fin] + 1e-300), algo


# Shapes for the packed-MFMA kernels with the batch in the matrix rows
# (bf16/fp16, stride 1, input and output widths up to 32): the 32-image
# kernel (C % 8 == 0, N >= 16) and the 16-image kernel (C % 16 == 0,
# N >= 8, one or two 16-column output groups).  A ragged last image group
# (N not a multiple of 16 or 32), ragged last row chunk (OH not a multiple
# of 7), the widest input (32 columns), FH != FW, a one-column filter,
# FW = 32 with PW = 16, several channel blocks (and channel-block counts
# that are not a multiple of the neighbour group), filters taller than the
# image, output widths of 13, 16, 17 and 32, and both padding extremes the
# kernels take.
BATCH_SHAPES = [
    (16, 28, 28, 16, 31, 31, 1, 15),
    (33, 14, 13, 24, 5, 5, 1, 2),
    (40, 12, 32, 8, 3, 7, 1, (1, 3)),
    (20, 20, 20, 16, 13, 13, 1, 6),
    (16, 9, 30, 8, 9, 1, 1, (4, 0)),
    (17, 8, 8, 8, 32, 32, 1, 16),
    (18, 30, 31, 8, 17, 17, 1, 8),
    (64, 7, 7, 32, 7, 7, 1, 3),
    (16, 11, 26, 8, 11, 27, 1, (0, 13)),
    (25, 14, 13, 48, 5, 5, 1, 2),
    (9, 30, 32, 64, 17, 17, 1, 8),
    (12, 10, 17, 16, 3, 31, 1, (1, 15)),
    (8, 16, 16, 32, 9, 9, 1, 4),
    (19, 9, 12, 80, 21, 11, 1, (10, 3)),
]


def _batch_imgs(s, img):
    """Images per instruction of the batch-packed plan when img (16 or 32)
    is asked for: the 16-image kernel where it applies, else the 32-image
    one, else None."""
    if img == 16 and s.c % 16 == 0 and s.n >= 8:
        return 16
    if s.c % 8 == 0 and s.n >= 16:
        return 32
    return None


@pytest.mark.parametrize("img", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data"])
@pytest.mark.parametrize("shape", BATCH_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_p{t[7]}")
def test_mfma_batch_parity(shape, op, dtype, img, monkeypatch):
    monkeypatch.setenv("DWC_MFMA_BATCH", "1")  # every filter height, not only AUTO's
    monkeypatch.setenv("DWC_MFMA_BATCH_IMG", str(img))
    s = _shape(shape)
    want_imgs = _batch_imgs(s, img)
    if want_imgs is None or (img == 32 and want_imgs != 32):
        pytest.skip("the batch-packed kernel asked for does not take this shape")
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT[dtype],
                    algo="mfma")
    d = dwc.plan_describe(p, OPS[op])
    assert " batch=1 " in d and f" imgs={want_imgs} " in d, d
    inp = make_inputs(s, dtype, seed=90 + sum(shape[:6]))
    want, mag = _want_mag(op, s, inp)
    log(f"case mfma batch {shape} {op} {dtype} imgs={want_imgs}")
    for algo in ("auto", "mfma"):
        got = _run(op, s, inp, algo)
        check_parity(got, want, mag, op, s, dtype, what=algo)


@pytest.mark.parametrize("shape", [(33, 14, 13, 24, 5, 5, 1, 2), (25, 14, 13, 48, 5, 5, 1, 2)],
                         ids=["imgs32", "imgs16"])
def test_mfma_batch_outputs_fully_overwritten(shape, monkeypatch):
    monkeypatch.setenv("DWC_MFMA_BATCH", "1")
    s = _shape(shape)
    inp = make_inputs(s, "bf16", seed=91)
    y = torch.full(s.y_shape(), float("nan"), device="cuda")
    dwc.fwd(to_device(inp.x), to_device(inp.w), 1, 2, out=y)
    dx = torch.full(s.x_shape(), float("nan"), device="cuda")
    dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (14, 13), 1, 2, out=dx)
    sync()
    for op, t in (("fwd", y), ("bwd_data", dx)):
        want, mag = _want_mag(op, s, inp)
        check_parity(t.double().cpu().numpy(), want, mag, op, s, "bf16", what=op)

"""GPU parity of the fp32 matrix-core forward-type kernel (fwd_mfma_f32)
against the float64 oracle: every element, forward and data gradient, each
tile width (2, 4 and 7 four-column tiles per wave) and each instantiated band
width, over shapes with ragged batches, rows, columns and channel blocks,
filters narrower than their band (zero taps), unequal and cropping padding,
images smaller than the filter, and outputs that must be overwritten
completely."""

import pytest

from dwc_inputs import make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import check_parity, dwc, log, sync, to_device  # noqa: E402
from test_parity_gpu import DT, OPS, _run, _shape, _want_mag  # noqa: E402

# (n, h, w, c, fh, fw, stride, pad)
F32M_SHAPES = [
    (2, 14, 14, 32, 13, 13, 1, 6),
    (3, 9, 23, 16, 17, 17, 1, 8),
    (1, 28, 28, 48, 31, 31, 1, 15),
    (2, 30, 57, 16, 21, 21, 1, 10),
    (2, 11, 13, 32, 9, 13, 1, (4, 6)),
    (1, 7, 7, 16, 31, 31, 1, 15),
    (2, 16, 16, 64, 27, 27, 1, 13),
    (2, 12, 20, 16, 5, 11, 1, (2, 3)),
    (1, 10, 10, 16, 13, 13, 1, 14),
    (2, 20, 9, 32, 15, 3, 1, (7, 1)),
    (5, 6, 40, 16, 1, 31, 1, (0, 15)),
    (1, 40, 8, 16, 64, 7, 1, (31, 3)),
    (3, 56, 56, 16, 31, 31, 1, 15),
]


def _ids(t):
    return "x".join(map(str, t[:6])) + f"_p{t[7]}"


# batches of 4 and more: the images kernel (fwd_mfma_f32n), ragged last
# image groups included
F32N_SHAPES = [
    (4, 14, 14, 32, 13, 13, 1, 6),
    (6, 9, 23, 16, 17, 17, 1, 8),
    (5, 28, 28, 16, 31, 31, 1, 15),
    (4, 10, 57, 16, 21, 21, 1, 10),
    (7, 12, 20, 16, 5, 11, 1, (2, 3)),
    (4, 10, 10, 16, 13, 13, 1, 14),
    (9, 7, 7, 16, 31, 31, 1, 15),
    (4, 40, 8, 16, 64, 7, 1, (31, 3)),
    (5, 6, 40, 16, 1, 31, 1, (0, 15)),
]


@pytest.mark.parametrize("img", [0, 1])
@pytest.mark.parametrize("tile", ["auto", "2", "4", "7"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data"])
@pytest.mark.parametrize("shape", F32M_SHAPES + F32N_SHAPES, ids=_ids)
def test_mfma_f32_parity(shape, op, tile, img, monkeypatch):
    s = _shape(shape)
    if img and (s.n < 4 or tile == "7"):
        pytest.skip("the images kernel takes batches of 4 and more, 2 or 4 tiles per wave")
    if tile != "auto":
        monkeypatch.setenv("DWC_MFMA_F32_T", tile)
    monkeypatch.setenv("DWC_MFMA_F32_IMG", str(img))
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT["f32"],
                    algo="mfma")
    d = dwc.plan_describe(p, OPS[op])
    assert " f32=1 " in d and f" img={img} " in d, d
    if tile != "auto":
        assert f" t={tile} " in d, d
    inp = make_inputs(s, "f32", seed=70 + sum(shape[:6]))
    want, mag = _want_mag(op, s, inp)
    log(f"case mfma f32 {shape} {op} t={tile}: {d}")
    got = _run(op, s, inp, "mfma")
    check_parity(got, want, mag, op, s, "f32", what=f"t={tile}")


@pytest.mark.parametrize("shape", [(2, 14, 14, 32, 13, 13, 1, 6), (2, 30, 57, 16, 21, 21, 1, 10),
                                   (5, 14, 14, 32, 13, 13, 1, 6), (6, 30, 57, 16, 21, 21, 1, 10)],
                         ids=_ids)
def test_mfma_f32_outputs_fully_overwritten(shape):
    s = _shape(shape)
    inp = make_inputs(s, "f32", seed=71)
    pad = (s.pad_h, s.pad_w)
    y = torch.full(s.y_shape(), float("nan"), device="cuda")
    dwc.fwd(to_device(inp.x), to_device(inp.w), 1, pad, out=y, algo="mfma")
    dx = torch.full(s.x_shape(), float("nan"), device="cuda")
    dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (s.h, s.w), 1, pad, out=dx, algo="mfma")
    sync()
    for op, t in (("fwd", y), ("bwd_data", dx)):
        want, mag = _want_mag(op, s, inp)
        check_parity(t.double().cpu().numpy(), want, mag, op, s, "f32", what=op)


@pytest.mark.parametrize("n", [2, 6])
def test_mfma_f32_deterministic(n):
    """Overlapping column groups write the same values: two runs agree bit
    for bit."""
    s = _shape((n, 30, 57, 16, 21, 21, 1, 10))
    inp = make_inputs(s, "f32", seed=72)
    x, w = to_device(inp.x), to_device(inp.w)
    a = dwc.fwd(x, w, 1, 10, algo="mfma")
    b = dwc.fwd(x, w, 1, 10, algo="mfma")
    sync()
    assert torch.equal(a, b)


# (n, h, w, c, fh, fw, stride, pad): the filter gradient's column tiles
# (FW 1 .. 32), output widths of each column-group size and wider than one
# group, filter heights up to 32, cropping padding
F32W_SHAPES = [
    (2, 14, 14, 32, 13, 13, 1, 6),
    (3, 9, 23, 16, 17, 17, 1, 8),
    (1, 28, 28, 48, 31, 31, 1, 15),
    (2, 10, 70, 16, 21, 21, 1, 10),
    (2, 11, 13, 32, 9, 13, 1, (4, 6)),
    (1, 7, 7, 16, 31, 31, 1, 15),
    (2, 12, 20, 16, 5, 11, 1, (2, 3)),
    (1, 10, 10, 16, 13, 13, 1, 14),
    (2, 20, 9, 32, 15, 3, 1, (7, 1)),
    (5, 6, 40, 16, 1, 31, 1, (0, 15)),
    (1, 40, 8, 16, 32, 32, 1, (16, 16)),
    (3, 30, 30, 16, 27, 27, 1, 13),
]


@pytest.mark.parametrize("split", [0, 1, 7])
@pytest.mark.parametrize("shape", F32W_SHAPES, ids=_ids)
def test_mfma_f32_wgrad_parity(shape, split):
    s = _shape(shape)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT["f32"],
                    algo="mfma", wgrad_split=split)
    d = dwc.plan_describe(p, OPS["bwd_filter"])
    assert d.startswith("bwd_filter mfma dt=f32") and " f32=1 " in d, d
    inp = make_inputs(s, "f32", seed=80 + sum(shape[:6]))
    want, mag = _want_mag("bwd_filter", s, inp)
    log(f"case mfma f32 wgrad {shape} split={split}: {d}")
    got = _run("bwd_filter", s, inp, "mfma", wgrad_split=split)
    check_parity(got, want, mag, "bwd_filter", s, "f32", what=f"split={split}")


# 16-bit operands on the same filter-gradient kernel, widened to fp32 as
# they are loaded: inputs wider than 64 (past the packed 16-bit kernel) and
# 56-wide ones with 13x13 filters (past its LDS budget); column tiles from
# 1 to 8, two column groups, cropping padding
F32W16_SHAPES = [
    (2, 10, 70, 16, 21, 21, 1, 10),
    (3, 9, 66, 32, 13, 13, 1, 6),
    (2, 12, 80, 16, 5, 11, 1, (2, 3)),
    (1, 8, 72, 48, 1, 31, 1, (0, 15)),
    (2, 56, 56, 16, 13, 13, 1, 6),
    (1, 40, 65, 16, 32, 32, 1, (16, 16)),
    (2, 30, 100, 16, 17, 9, 1, (8, 4)),
]


@pytest.mark.parametrize("split", [0, 7])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", F32W16_SHAPES, ids=_ids)
def test_mfma_f32_wgrad_16bit_parity(shape, dtype, split):
    s = _shape(shape)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT[dtype],
                    algo="mfma", wgrad_split=split)
    d = dwc.plan_describe(p, OPS["bwd_filter"])
    assert d.startswith(f"bwd_filter mfma dt={dtype}") and " f32=1 " in d, d
    inp = make_inputs(s, dtype, seed=90 + sum(shape[:6]))
    want, mag = _want_mag("bwd_filter", s, inp)
    log(f"case mfma f32 wgrad {dtype} {shape} split={split}: {d}")
    got = _run("bwd_filter", s, inp, "mfma", wgrad_split=split)
    check_parity(got, want, mag, "bwd_filter", s, dtype, what=f"split={split}")


# 16-bit operands on the rows forward-type kernel (widened on load): outputs
# wider than 64 (past the packed 16-bit kernels), each band width and tile
# width, the flipped data gradient, ragged rows and columns
F32M16_SHAPES = [
    (2, 10, 70, 16, 13, 13, 1, 6),
    (1, 12, 80, 32, 17, 17, 1, 8),
    (2, 9, 66, 16, 21, 11, 1, (10, 5)),
    (1, 20, 90, 16, 27, 27, 1, 13),
    (1, 33, 67, 48, 31, 31, 1, 15),
]


@pytest.mark.parametrize("tile", ["auto", "2", "4", "7"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", F32M16_SHAPES, ids=_ids)
def test_mfma_f32_16bit_parity(shape, dtype, op, tile, monkeypatch):
    if tile != "auto":
        monkeypatch.setenv("DWC_MFMA_F32_T", tile)
    s = _shape(shape)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT[dtype],
                    algo="mfma")
    d = dwc.plan_describe(p, OPS[op])
    assert f" mfma dt={dtype} " in d and " f32=1 " in d and " img=0 " in d, d
    inp = make_inputs(s, dtype, seed=95 + sum(shape[:6]))
    want, mag = _want_mag(op, s, inp)
    log(f"case mfma f32 {dtype} {op} {shape} tile={tile}: {d}")
    got = _run(op, s, inp, "mfma")
    check_parity(got, want, mag, op, s, dtype, what=f"tile={tile}")


def test_mfma_f32_wgrad_deterministic():
    s = _shape((3, 30, 30, 16, 27, 27, 1, 13))
    inp = make_inputs(s, "f32", seed=81)
    x, dy = to_device(inp.x), to_device(inp.dy)
    a = dwc.bwd_filter(x, dy, (27, 27), 1, 13, algo="mfma")
    b = dwc.bwd_filter(x, dy, (27, 27), 1, 13, algo="mfma")
    sync()
    assert torch.equal(a, b)

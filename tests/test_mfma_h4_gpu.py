"""GPU parity of the 16-bit forward-type kernel on the 4x4x4 matrix
instructions (fwd_mfma_h4n) against the float64 oracle: every element,
forward and data gradient, bf16 and fp16, both tile widths (4 and 7
four-column tiles per wave) and each instantiated band width, over shapes
with ragged image groups, rows, columns and channel blocks, filters
narrower than their band (zero taps), unequal and cropping padding, images
smaller than the filter, windows that reach past the image, and outputs
that must be overwritten completely."""

import pytest

from dwc_inputs import make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import check_parity, dwc, log, sync, to_device  # noqa: E402
from test_parity_gpu import DT, OPS, _run, _shape, _want_mag  # noqa: E402

# (n, h, w, c, fh, fw, stride, pad)
H4_SHAPES = [
    (4, 28, 28, 32, 13, 13, 1, 6),       # one 28-column group, no range test
    (5, 14, 14, 16, 13, 13, 1, 6),       # ragged image group, 16 columns for 14
    (3, 9, 23, 16, 9, 9, 1, 4),          # fewer than 4 images
    (2, 30, 57, 16, 17, 17, 1, 8),       # several column groups, the last right-aligned
    (6, 11, 13, 32, 9, 13, 1, (4, 6)),   # FH != FW
    (4, 12, 20, 16, 5, 11, 1, (2, 3)),   # band wider than the filter, unequal padding
    (1, 10, 10, 16, 13, 13, 1, 14),      # padding beyond F - 1 (cropping data gradient)
    (4, 20, 9, 32, 15, 3, 1, (7, 1)),    # three-column filter
    (8, 7, 7, 16, 13, 13, 1, 6),         # image smaller than the filter
    (4, 56, 56, 16, 13, 13, 1, 6),       # two 28-column groups
    (3, 14, 8, 16, 20, 7, 1, (10, 3)),   # filter taller than the image
    (4, 30, 30, 16, 13, 13, 1, 6),       # edge windows reaching past the image
    (9, 17, 26, 48, 13, 13, 1, 6),       # three channel blocks, ragged everything
]


def _ids(t):
    return "x".join(map(str, t[:6])) + f"_p{t[7]}"


@pytest.mark.parametrize("tile", ["auto", "4", "7"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["fwd", "bwd_data"])
@pytest.mark.parametrize("shape", H4_SHAPES, ids=_ids)
def test_mfma_h4_parity(shape, op, dtype, tile, monkeypatch):
    s = _shape(shape)
    monkeypatch.setenv("DWC_MFMA_H4", "1")
    if tile != "auto":
        monkeypatch.setenv("DWC_MFMA_H4_T", tile)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT[dtype],
                    algo="mfma")
    d = dwc.plan_describe(p, OPS[op])
    assert " h4=1 " in d, d
    if tile != "auto":
        assert f" t={tile} " in d, d
    inp = make_inputs(s, dtype, seed=170 + sum(shape[:6]))
    want, mag = _want_mag(op, s, inp)
    log(f"case mfma h4 {shape} {op} {dtype} t={tile}: {d}")
    got = _run(op, s, inp, "mfma")
    check_parity(got, want, mag, op, s, dtype, what=f"t={tile}")


@pytest.mark.parametrize("shape", [(5, 14, 14, 32, 13, 13, 1, 6), (2, 30, 57, 16, 17, 17, 1, 8),
                                   (4, 28, 28, 16, 13, 13, 1, 6)], ids=_ids)
def test_mfma_h4_outputs_fully_overwritten(shape, monkeypatch):
    monkeypatch.setenv("DWC_MFMA_H4", "1")
    s = _shape(shape)
    inp = make_inputs(s, "bf16", seed=171)
    pad = (s.pad_h, s.pad_w)
    y = torch.full(s.y_shape(), float("nan"), device="cuda")
    dwc.fwd(to_device(inp.x), to_device(inp.w), 1, pad, out=y, algo="mfma")
    dx = torch.full(s.x_shape(), float("nan"), device="cuda")
    dwc.bwd_data(to_device(inp.dy), to_device(inp.w), (s.h, s.w), 1, pad, out=dx, algo="mfma")
    sync()
    for op, t in (("fwd", y), ("bwd_data", dx)):
        want, mag = _want_mag(op, s, inp)
        check_parity(t.double().cpu().numpy(), want, mag, op, s, "bf16", what=op)


@pytest.mark.parametrize("tile", ["4", "7"])
def test_mfma_h4_deterministic(tile, monkeypatch):
    """The last column group overlaps the one before it and groups a
    column's taps differently; only one of them writes each column, so
    repeated runs agree bit for bit."""
    monkeypatch.setenv("DWC_MFMA_H4", "1")
    monkeypatch.setenv("DWC_MFMA_H4_T", tile)
    s = _shape((6, 30, 57, 16, 17, 17, 1, 8))
    inp = make_inputs(s, "f16", seed=172)
    x, w = to_device(inp.x), to_device(inp.w)
    a = dwc.fwd(x, w, 1, 8, algo="mfma")
    for _ in range(4):
        b = dwc.fwd(x, w, 1, 8, algo="mfma")
        sync()
        assert torch.equal(a, b)

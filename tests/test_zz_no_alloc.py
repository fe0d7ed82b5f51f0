"""dwc_bwd_filter_noalloc: the filter gradient through the entry point that
allocates nothing (slice partials in the library's fixed per-device
scratch), checked against dwc_bwd_filter with a caller-owned workspace and
against the float64 oracle, on consecutive calls of different sizes."""

import numpy as np
import pytest

import oracle
from dwc_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import check_parity, dwc, log, sync, to_device  # noqa: E402

DT = {"f32": dwc.F32, "bf16": dwc.BF16, "f16": dwc.F16, "e4m3": dwc.FP8_E4M3}

# (first call, second call with a smaller input): the sweep kernels, the
# register-window kernels, the packed-MFMA kernels (16-bit and fp8 operands)
PAIRS = [
    ("f32", (8, 56, 56, 128, 7, 7, 1, 3), (2, 20, 20, 64, 7, 7, 1, 3)),
    ("f32", (8, 28, 28, 256, 13, 13, 1, 6), (1, 9, 9, 16, 13, 13, 1, 6)),
    ("bf16", (16, 28, 28, 512, 13, 13, 1, 6), (2, 14, 14, 32, 5, 5, 1, 2)),
    ("f16", (8, 28, 28, 256, 31, 31, 1, 15), (3, 12, 12, 16, 3, 3, 1, 1)),
    ("e4m3", (8, 28, 28, 512, 13, 13, 1, 6), (2, 10, 10, 16, 3, 3, 1, 1)),
]


def _shape(t):
    n, h, w, c, fh, fw, s, p = t
    return Shape(n, h, w, c, fh, fw, s, s, p, p)


def _vals(op):
    if op.dtype in oracle.FP8_FORMATS:
        return oracle.fp8_decode(op.stored, op.dtype)
    return op.values


def _oracle(s, inp):
    a, b = _vals(inp.x), _vals(inp.dy)
    f = lambda u, v: oracle.bwd_filter(u, v, (s.fh, s.fw), (s.stride_h, s.stride_w),
                                       (s.pad_h, s.pad_w))
    return f(a, b), f(np.abs(a), np.abs(b))


def _both(s, inp, wgrad_split=0):
    x, dy = to_device(inp.x), to_device(inp.dy)
    st, pd = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    out = torch.full(s.w_shape(), float("nan"), device="cuda")
    before = torch.cuda.memory_allocated()
    dwc.bwd_filter_noalloc(x, dy, (s.fh, s.fw), st, pd, out=out, wgrad_split=wgrad_split)
    assert torch.cuda.memory_allocated() == before
    ref = dwc.bwd_filter(x, dy, (s.fh, s.fw), st, pd, wgrad_split=wgrad_split)
    sync()
    return out.double().cpu().numpy(), ref.double().cpu().numpy()


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-k{p[1][4]}")
def test_noalloc_two_calls(pair):
    dtype, big, small = pair
    for t in (big, small):
        s = _shape(t)
        log(f"case noalloc {dtype} {t}")
        p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, (s.pad_h, s.pad_w), dtype=DT[dtype])
        assert dwc.workspace_size(p) <= dwc.NOALLOC_SCRATCH_BYTES
        inp = make_inputs(s, dtype, seed=100 + sum(t[:6]))
        got, ref = _both(s, inp)
        # the automatic split fits the scratch: same kernels, same order
        np.testing.assert_array_equal(got, ref)
        want, mag = _oracle(s, inp)
        check_parity(got, want, mag, "bwd_filter", s, dtype, what=f"noalloc {t}")


def test_noalloc_narrows_a_split_that_does_not_fit():
    """Partials of the automatic split exceed the scratch (the sweep kernels
    on a wide, shallow batch with many channels need 40.5 MiB): the call
    takes a split whose partials fit (here the one-output-per-lane kernels,
    since the sweep cannot slice more coarsely) and still gives the
    oracle's result; a split the caller sets that does not fit is rejected
    before any launch."""
    t = (16, 9, 112, 2048, 9, 9, 1, 4)
    s = _shape(t)
    p = dwc.problem(s.n, s.h, s.w, s.c, s.fh, s.fw, 1, 4)
    assert dwc.workspace_size(p) > dwc.NOALLOC_SCRATCH_BYTES
    inp = make_inputs(s, "f32", seed=7)
    log(f"case noalloc narrowed {t}")
    got, ref = _both(s, inp)
    want, mag = _oracle(s, inp)
    check_parity(got, want, mag, "bwd_filter", s, "f32", what="noalloc narrowed")
    check_parity(ref, want, mag, "bwd_filter", s, "f32", what="workspace")
    x, dy = to_device(inp.x), to_device(inp.dy)
    out = torch.zeros(s.w_shape(), device="cuda")
    with pytest.raises(dwc.DwcError) as e:
        dwc.bwd_filter_noalloc(x, dy, (9, 9), 1, 4, out=out, wgrad_split=16)
    assert e.value.status == 4  # DWC_ERR_WORKSPACE
    sync()
    assert torch.count_nonzero(out).item() == 0


def test_noalloc_empty_batch_and_bad_calls():
    x = torch.zeros((0, 8, 8, 16), device="cuda")
    dw = torch.full((3, 3, 16), 7.0, device="cuda")
    dwc.bwd_filter_noalloc(x, x, (3, 3), 1, 1, out=dw)
    sync()
    assert torch.count_nonzero(dw).item() == 0
    p = dwc.problem(1, 8, 8, 16, 3, 3, 1, 1)
    with pytest.raises(dwc.DwcError):  # NULL operands
        dwc.bwd_filter_noalloc_ptr(p, 0, 0, dw.data_ptr())

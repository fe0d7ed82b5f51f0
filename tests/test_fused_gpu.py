"""GPU parity of the fused-prologue forward (Flash-DWC §5.2): Y =
DWC(act(X * scale + shift), W) against the oracle, for both kernel families
(the row sweep at stride 1 with square filters, the row-tile kernel at
stride 2 and for other filters), every activation and operand dtype,
unequal padding, ragged channel blocks and image borders."""

import numpy as np
import pytest

import oracle
from dwc_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import TOL, dwc, log, rel_l2, sync, to_device  # noqa: E402

# (n, h, w, c, fh, fw, stride, pad)
FUSED_SHAPES = [
    (2, 14, 14, 64, 3, 3, 1, 1),       # sweep
    (1, 17, 19, 70, 5, 5, 1, 2),       # sweep, ragged channels
    (2, 20, 21, 128, 7, 7, 1, 3),      # sweep
    (1, 16, 13, 64, 9, 9, 1, (2, 4)),  # sweep, unequal padding
    (2, 20, 20, 64, 7, 7, 2, 3),       # row tiles, stride 2
    (1, 15, 17, 96, 3, 3, 2, 1),       # row tiles, stride 2
    (1, 12, 15, 64, 5, 3, 1, (2, 1)),  # row tiles, non-square filter
    (1, 30, 11, 64, 13, 9, 1, (6, 4)), # row tiles, filter rows in chunks
    (1, 9, 9, 8, 9, 9, 2, 0),          # no padding, C < 64
    (2, 13, 14, 64, 4, 4, 1, (1, 2)),  # even width on the 5-wide body
    (1, 14, 17, 40, 3, 8, 2, (1, 3)),  # 8 on the 9-wide body, stride 2
    (1, 10, 12, 64, 1, 1, 1, 0),       # 1x1 on the 3-wide body
]


def _shape(t):
    n, h, w, c, fh, fw, s, p = t
    ph, pw = (p, p) if isinstance(p, int) else p
    return Shape(n, h, w, c, fh, fw, s, s, ph, pw)


@pytest.mark.parametrize("act", ["none", "relu", "relu6", "silu"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", FUSED_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_s{t[6]}_p{t[7]}")
def test_fused_forward_parity(shape, dtype, act):
    s = _shape(shape)
    inp = make_inputs(s, dtype, seed=110 + sum(shape[:6]))
    r = np.random.default_rng(7 + s.c)
    scale = (1.0 + 0.5 * r.standard_normal(s.c)).astype(np.float32)
    shift = (0.5 * r.standard_normal(s.c)).astype(np.float32)
    stride, pad = (s.stride_h, s.stride_w), (s.pad_h, s.pad_w)
    want = oracle.fwd_fused(inp.x.values, scale.astype(np.float64), shift.astype(np.float64),
                            act, inp.w.values, stride, pad)
    log(f"case fused {shape} {dtype} {act}")
    sc, sh = torch.from_numpy(scale).cuda(), torch.from_numpy(shift).cuda()
    for algo in ("auto", "direct"):
        got = dwc.fwd_fused(to_device(inp.x), to_device(inp.w), sc, sh, act, stride, pad,
                            algo=algo)
        sync()
        got = got.double().cpu().numpy()
        assert got.shape == want.shape
        assert np.all(np.isfinite(got))
        assert rel_l2(got, want) <= TOL[dtype], (algo, rel_l2(got, want))


def test_fused_overwrites_output_and_keeps_padding_zero():
    """A shift that makes act(shift) large: outputs at the image border only
    see the taps inside the image (the padding of X' is zero)."""
    s = _shape((1, 9, 9, 64, 7, 7, 1, 3))
    inp = make_inputs(s, "f32", seed=9)
    scale = np.full(64, 0.25, np.float32)
    shift = np.full(64, 3.0, np.float32)
    y = torch.full(s.y_shape(), float("nan"), device="cuda")
    dwc.fwd_fused(to_device(inp.x), to_device(inp.w), torch.from_numpy(scale).cuda(),
                  torch.from_numpy(shift).cuda(), "relu6", 1, 3, out=y)
    sync()
    assert torch.isfinite(y).all().item()
    want = oracle.fwd_fused(inp.x.values, scale.astype(np.float64), shift.astype(np.float64),
                            "relu6", inp.w.values, 1, 3)
    assert rel_l2(y.double().cpu().numpy(), want) <= TOL["f32"]

"""GPU parity of the hybrid-accumulation filter gradient (Flash-DWC §5.1:
fp16 sub-unit sums merged in fp32; fp16 operands, DWC_ALGO_HYBRID) against
the oracle, within the half-precision budget of 3e-3, including one
full-size batch where each tap sums 200704 products."""

import numpy as np
import pytest

import oracle
from dwc_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU too; skipped there
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import TOL, dwc, gather, log, rel_l2, sample_index, sync, to_device  # noqa: E402

HYB_SHAPES = [
    (2, 14, 14, 64, 3, 3, 1, 1),
    (2, 17, 19, 70, 5, 5, 1, 2),
    (3, 20, 21, 128, 7, 7, 1, 3),
    (1, 16, 13, 64, 9, 9, 1, (2, 4)),
    (2, 30, 28, 64, 3, 3, 1, (0, 1)),
    (1, 9, 9, 8, 7, 7, 1, 0),
]


def _shape(t):
    n, h, w, c, fh, fw, s, p = t
    ph, pw = (p, p) if isinstance(p, int) else p
    return Shape(n, h, w, c, fh, fw, s, s, ph, pw)


def _run(s, inp, split=0):
    return dwc.bwd_filter(to_device(inp.x), to_device(inp.dy), (s.fh, s.fw),
                          (s.stride_h, s.stride_w), (s.pad_h, s.pad_w), wgrad_split=split,
                          algo="hybrid")


@pytest.mark.parametrize("rows", [0, 2, 5])
@pytest.mark.parametrize("shape", HYB_SHAPES,
                         ids=lambda t: "x".join(map(str, t[:6])) + f"_p{t[7]}")
def test_hybrid_wgrad_parity(shape, rows, monkeypatch):
    if rows:
        monkeypatch.setenv("DWC_SWEEP_ROWS", str(rows))
    s = _shape(shape)
    inp = make_inputs(s, "f16", seed=130 + sum(shape[:6]))
    want = oracle.bwd_filter(inp.x.values, inp.dy.values, (s.fh, s.fw), (1, 1),
                             (s.pad_h, s.pad_w))
    log(f"case hybrid {shape} rows={rows}")
    got = _run(s, inp)
    sync()
    g = got.double().cpu().numpy()
    err = rel_l2(g, want)
    log(f"  rel_l2 = {err:.3e}")
    assert err <= TOL["f16"], err
    again = _run(s, inp)
    sync()
    assert np.array_equal(g, again.double().cpu().numpy())  # deterministic


def test_hybrid_wgrad_full_size_long_accumulation():
    """N=64, 56x56, C=128, 7x7: every tap sums N*OH*OW = 200704 products,
    in fp16 sub-units of at most 63 merged in fp32."""
    s = _shape((64, 56, 56, 128, 7, 7, 1, 3))
    inp = make_inputs(s, "f16", seed=0)
    got = _run(s, inp)
    sync()
    rng = np.random.default_rng(2)
    idx = sample_index(s.w_shape(), 256, rng)
    want = oracle.bwd_filter_at(inp.x.values, inp.dy.values, (7, 7), idx, (1, 1), (3, 3))
    err = rel_l2(gather(got, idx), want)
    log(f"full-size hybrid rel_l2 = {err:.3e}")
    assert err <= TOL["f16"], err
    ref = dwc.bwd_filter(to_device(inp.x), to_device(inp.dy), (7, 7), 1, 3, algo="direct")
    sync()
    assert rel_l2(got.double().cpu().numpy(), ref.double().cpu().numpy()) <= TOL["f16"]

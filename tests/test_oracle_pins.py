"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties the oracle to something fixed by the pages or by mathematics:
hand-worked examples of the definition (``tests/golden``), a second
formulation (the im2col -> per-channel GEMV view of Flash-DWC (TACO) §2.1,
Fig. 1), special cases with exact answers, invariants, the adjoint identities
that define the two gradients (§5.1), finite differences, and textbook
library routines.  The mutation tests at the end plant plausible mistakes in a
copy of the oracle's C source and check that the pins catch every one.
"""

import json
import os
import re

import numpy as np
import pytest

import oracle
from dwc_inputs import Shape, make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _img(a):
    """One-image, one-channel N x H x W x C array from an H x W list."""
    return np.asarray(a, dtype=np.float64)[None, :, :, None]


def _filt(a):
    return np.asarray(a, dtype=np.float64)[:, :, None]


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- golden ----

def check_golden(orc):
    fw = _load("fwd_hand_examples.json")
    for case in fw["cases"]:
        y = orc.fwd(_img(case["x_hw"]), _filt(case["w_hw"]), case["stride"], case["pad"])
        np.testing.assert_array_equal(y[0, :, :, 0], np.asarray(case["y_hw"], float),
                                      err_msg=case["name"])
    bw = _load("bwd_hand_examples.json")
    for case in bw["bwd_data"]:
        dx = orc.bwd_data(_img(case["dy_hw"]), _filt(case["w_hw"]), case["in_hw"],
                          case["stride"], case["pad"])
        np.testing.assert_array_equal(dx[0, :, :, 0], np.asarray(case["dx_hw"], float),
                                      err_msg=case["name"])
    for case in bw["bwd_filter"]:
        dw = orc.bwd_filter(_img(case["x_hw"]), _img(case["dy_hw"]), case["f_hw"],
                            case["stride"], case["pad"])
        np.testing.assert_array_equal(dw[:, :, 0], np.asarray(case["dw_hw"], float),
                                      err_msg=case["name"])


def test_golden_hand_examples():
    check_golden(oracle.get())


# ------------------------------------------------- second formulation -------

def im2col_gemv(x, w, stride, pad):
    """Flash-DWC (TACO) §2.1, Fig. 1: per channel, the unrolled input patches
    form a matrix and the unrolled filter a vector; Y is their product."""
    n, h, wd, c = x.shape
    fh, fw, _ = w.shape
    s, p = stride, pad
    xp = np.zeros((n, h + 2 * p, wd + 2 * p, c))
    xp[:, p:p + h, p:p + wd, :] = x
    oh = (h + 2 * p - fh) // s + 1
    ow = (wd + 2 * p - fw) // s + 1
    y = np.empty((n, oh, ow, c))
    for ch in range(c):
        vec = w[:, :, ch].reshape(-1)
        for b in range(n):
            mat = np.array([xp[b, i * s:i * s + fh, j * s:j * s + fw, ch].reshape(-1)
                            for i in range(oh) for j in range(ow)])
            y[b, :, :, ch] = (mat @ vec).reshape(oh, ow)
    return y


def _tiny_cases(count=40, seed=1):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        n = int(rng.integers(1, 3))
        h, w = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        c = int(rng.choice([1, 3]))
        f = int(rng.choice([1, 2, 3, 5]))
        s = int(rng.choice([1, 2]))
        p = int(rng.integers(0, 3))
        if h + 2 * p < f or w + 2 * p < f:
            continue
        cases.append((n, h, w, c, f, s, p))
    return cases


@pytest.mark.parametrize("case", _tiny_cases())
def test_fwd_matches_im2col_gemv(case):
    n, h, w, c, f, s, p = case
    rng = np.random.default_rng(hash(case) % 2**32)
    x = rng.standard_normal((n, h, w, c))
    wt = rng.standard_normal((f, f, c))
    np.testing.assert_allclose(oracle.fwd(x, wt, s, p), im2col_gemv(x, wt, s, p),
                               rtol=1e-13, atol=1e-13)


# ------------------------------------------------------ special cases -------

@pytest.mark.parametrize("s,p,f", [(1, 1, 3), (1, 2, 5), (2, 1, 3), (2, 3, 7), (1, 0, 2)])
def test_delta_filter_is_a_shift(s, p, f):
    """W = e_(i,j): Y[n,oh,ow,c] = Xz[n, oh*s-p+i, ow*s-p+j, c], exactly."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 9, 8, 3))
    for i in range(f):
        for j in range(f):
            w = np.zeros((f, f, 3))
            w[i, j, :] = 1.0
            y = oracle.fwd(x, w, s, p)
            xz = np.zeros((2, 9 + 2 * p + f, 8 + 2 * p + f, 3))
            xz[:, p:p + 9, p:p + 8, :] = x
            oh, ow = y.shape[1:3]
            want = xz[:, i:i + (oh - 1) * s + 1:s, j:j + (ow - 1) * s + 1:s, :]
            np.testing.assert_array_equal(y, want)


def test_centred_delta_is_identity():
    """With stride 1, 'same' padding p and the centred delta, Y equals X bitwise."""
    x = make_inputs(Shape(2, 11, 10, 5, 7, 7, 1, 1, 3, 3), "f32", seed=3).x.values
    w = np.zeros((7, 7, 5))
    w[3, 3, :] = 1.0
    np.testing.assert_array_equal(oracle.fwd(x, w, 1, 3), x.astype(np.float64))


def test_ones_input_closed_form():
    """X = 1: each output is the sum of the filter taps that land on the image
    (all taps in the interior)."""
    f, p, h = 5, 2, 9
    rng = np.random.default_rng(11)
    w = rng.standard_normal((f, f, 4))
    y = oracle.fwd(np.ones((1, h, h, 4)), w, 1, p)
    for oh in range(h):
        for ow in range(h):
            r0, r1 = max(0, p - oh), min(f, h + p - oh)
            c0, c1 = max(0, p - ow), min(f, h + p - ow)
            np.testing.assert_allclose(y[0, oh, ow], w[r0:r1, c0:c1].sum(axis=(0, 1)),
                                       rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y[0, 4, 4], w.sum(axis=(0, 1)), rtol=1e-14)


def test_linearity_and_channel_independence():
    rng = np.random.default_rng(5)
    x1 = rng.standard_normal((2, 8, 7, 6))
    x2 = rng.standard_normal((2, 8, 7, 6))
    w = rng.standard_normal((3, 5, 6))
    a, b = 0.75, -2.5
    lhs = oracle.fwd(a * x1 + b * x2, w, 1, (1, 2))
    rhs = a * oracle.fwd(x1, w, 1, (1, 2)) + b * oracle.fwd(x2, w, 1, (1, 2))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # depthwise: changing channel 2 of X changes only channel 2 of Y
    x3 = x1.copy()
    x3[..., 2] += rng.standard_normal(x3.shape[:3])
    y1, y3 = oracle.fwd(x1, w, 1, (1, 2)), oracle.fwd(x3, w, 1, (1, 2))
    keep = [c for c in range(6) if c != 2]
    np.testing.assert_array_equal(y1[..., keep], y3[..., keep])
    assert not np.array_equal(y1[..., 2], y3[..., 2])


def test_row_decomposition():
    """Flash-DWC (TACO) §3.3: a 2-D filter is FH 1-D rows; the 2-D result is
    the sum of FH 1-D DWCs, each on the input shifted down by the row index."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 9, 10, 3))
    w = rng.standard_normal((4, 3, 3))
    p = 1
    y = oracle.fwd(x, w, 1, p)
    acc = np.zeros_like(y)
    xz = np.zeros((1, 9 + 2 * p, 10 + 2 * p, 3))
    xz[:, p:p + 9, p:p + 10] = x
    oh, ow = y.shape[1:3]
    for r in range(4):
        rows = xz[:, r:r + oh, :, :]  # input rows used with filter row r
        for k in range(3):  # 1-D DWC along the width with the row's taps
            acc += rows[:, :, k:k + ow, :] * w[r, k, :]
    np.testing.assert_allclose(y, acc, rtol=1e-13, atol=1e-13)


def test_stride_two_subsamples_stride_one():
    x = make_inputs(Shape(2, 13, 12, 4, 5, 5, 1, 1, 2, 2), "f32", seed=4).x.values
    w = np.random.default_rng(4).standard_normal((5, 5, 4))
    y1 = oracle.fwd(x, w, 1, 2)
    y2 = oracle.fwd(x, w, 2, 2)
    np.testing.assert_array_equal(y2, y1[:, ::2, ::2, :])


def test_output_dims():
    assert oracle.output_dims(14, 14, 7, 7, 1, 3) == (14, 14)
    assert oracle.output_dims(56, 56, 7, 7, 2, 3) == (28, 28)
    assert oracle.output_dims(56, 56, 31, 31, 1, 15) == (56, 56)
    assert oracle.output_dims(7, 7, 31, 31, 1, 15) == (7, 7)
    assert oracle.output_dims(3, 3, 3, 3, 2, 1) == (2, 2)


# ------------------------------------------------------------ gradients -----

def _grad_cases():
    return [
        (2, 7, 6, 3, 3, 3, 1, 1, 1, 1),
        (1, 9, 9, 2, 5, 5, 1, 1, 2, 2),
        (2, 8, 9, 3, 3, 5, 2, 2, 1, 2),
        (1, 10, 7, 2, 4, 2, 2, 1, 0, 1),
        (3, 5, 5, 4, 7, 7, 1, 1, 3, 3),
        (1, 6, 11, 1, 1, 3, 3, 2, 0, 1),
    ]


@pytest.mark.parametrize("case", _grad_cases())
def test_bwd_data_is_adjoint(case):
    """<dY, fwd(X)> = <bwd_data(dY), X>: the data gradient is the adjoint."""
    n, h, w_, c, fh, fw, sh, sw, ph, pw = case
    rng = np.random.default_rng(sum(case))
    x = rng.standard_normal((n, h, w_, c))
    w = rng.standard_normal((fh, fw, c))
    y = oracle.fwd(x, w, (sh, sw), (ph, pw))
    dy = rng.standard_normal(y.shape)
    dx = oracle.bwd_data(dy, w, (h, w_), (sh, sw), (ph, pw))
    lhs, rhs = np.vdot(dy, y), np.vdot(dx, x)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("case", _grad_cases())
def test_bwd_filter_is_adjoint(case):
    """<dY, fwd(X, W)> = <bwd_filter(X, dY), W>."""
    n, h, w_, c, fh, fw, sh, sw, ph, pw = case
    rng = np.random.default_rng(100 + sum(case))
    x = rng.standard_normal((n, h, w_, c))
    w = rng.standard_normal((fh, fw, c))
    y = oracle.fwd(x, w, (sh, sw), (ph, pw))
    dy = rng.standard_normal(y.shape)
    dw = oracle.bwd_filter(x, dy, (fh, fw), (sh, sw), (ph, pw))
    lhs, rhs = np.vdot(dy, y), np.vdot(dw, w)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("f,p", [(3, 1), (5, 2), (3, 0), (7, 3), (4, 2)])
def test_bwd_data_is_rotated_forward(f, p):
    """Flash-DWC (TACO) §5.1: for stride 1 the data gradient is the forward
    DWC of dY with the filter turned by 180 degrees (padding f-1-p)."""
    rng = np.random.default_rng(f * 10 + p)
    h, wd, c = 9, 8, 3
    w = rng.standard_normal((f, f, c))
    oh, ow = oracle.output_dims(h, wd, f, f, 1, p)
    dy = rng.standard_normal((2, oh, ow, c))
    dx = oracle.bwd_data(dy, w, (h, wd), 1, p)
    rot = w[::-1, ::-1, :]
    np.testing.assert_allclose(dx, oracle.fwd(dy, rot, 1, f - 1 - p), rtol=1e-12, atol=1e-12)


def test_bwd_filter_finite_differences():
    """L(W) = <dY, fwd(X, W)> is linear in W, so a central difference with any
    step is exact up to rounding: (L(W+e_k) - L(W-e_k)) / 2 = dW_k."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 8, 9, 3))
    w = rng.standard_normal((5, 3, 3))
    dy = rng.standard_normal(oracle.fwd(x, w, (2, 1), (2, 1)).shape)
    dw = oracle.bwd_filter(x, dy, (5, 3), (2, 1), (2, 1))
    for k in [(0, 0, 0), (4, 2, 1), (2, 1, 2), (1, 0, 1), (3, 2, 0)]:
        e = np.zeros_like(w)
        e[k] = 1.0
        lp = np.vdot(dy, oracle.fwd(x, w + e, (2, 1), (2, 1)))
        lm = np.vdot(dy, oracle.fwd(x, w - e, (2, 1), (2, 1)))
        assert abs((lp - lm) / 2 - dw[k]) <= 1e-10 * max(1.0, abs(dw[k]))


# --------------------------------------------------- library routines -------

torch = pytest.importorskip("torch")


def _torch_ref(x, w, dy, stride, pad):
    """Grouped convolution (groups = C) in float64 on the CPU, with autograd
    for both gradients: a textbook routine independent of the oracle."""
    xt = torch.tensor(x.transpose(0, 3, 1, 2), dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w.transpose(2, 0, 1)[:, None], dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.conv2d(xt, wt, stride=stride, padding=pad, groups=x.shape[3])
    g = torch.tensor(dy.transpose(0, 3, 1, 2), dtype=torch.float64)
    y.backward(g)
    return (y.detach().numpy().transpose(0, 2, 3, 1),
            xt.grad.numpy().transpose(0, 2, 3, 1),
            wt.grad.numpy()[:, 0].transpose(1, 2, 0))


@pytest.mark.parametrize("case", _grad_cases())
def test_against_torch_grouped_conv(case):
    n, h, w_, c, fh, fw, sh, sw, ph, pw = case
    rng = np.random.default_rng(300 + sum(case))
    x = rng.standard_normal((n, h, w_, c))
    w = rng.standard_normal((fh, fw, c))
    y = oracle.fwd(x, w, (sh, sw), (ph, pw))
    dy = rng.standard_normal(y.shape)
    ty, tdx, tdw = _torch_ref(x, w, dy, (sh, sw), (ph, pw))
    np.testing.assert_allclose(y, ty, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.bwd_data(dy, w, (h, w_), (sh, sw), (ph, pw)), tdx,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.bwd_filter(x, dy, (fh, fw), (sh, sw), (ph, pw)), tdw,
                               rtol=1e-12, atol=1e-12)


def test_against_scipy_correlate2d():
    signal = pytest.importorskip("scipy.signal")
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1, 12, 10, 3))
    w = rng.standard_normal((5, 3, 3))
    y = oracle.fwd(x, w, 1, (2, 1))
    for c in range(3):
        xz = np.pad(x[0, :, :, c], ((2, 2), (1, 1)))
        np.testing.assert_allclose(y[0, :, :, c], signal.correlate2d(xz, w[:, :, c], "valid"),
                                   rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ sampled forms -------

@pytest.mark.parametrize("case", _grad_cases())
def test_sampled_forms_match_full(case):
    n, h, w_, c, fh, fw, sh, sw, ph, pw = case
    rng = np.random.default_rng(500 + sum(case))
    x = rng.standard_normal((n, h, w_, c))
    w = rng.standard_normal((fh, fw, c))
    y = oracle.fwd(x, w, (sh, sw), (ph, pw))
    dy = rng.standard_normal(y.shape)
    dx = oracle.bwd_data(dy, w, (h, w_), (sh, sw), (ph, pw))
    dw = oracle.bwd_filter(x, dy, (fh, fw), (sh, sw), (ph, pw))
    iy = np.argwhere(np.ones(y.shape, bool))
    ix = np.argwhere(np.ones(dx.shape, bool))
    iw = np.argwhere(np.ones(dw.shape, bool))
    np.testing.assert_allclose(oracle.fwd_at(x, w, iy, (sh, sw), (ph, pw)), y.reshape(-1),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.bwd_data_at(dy, w, (h, w_), ix, (sh, sw), (ph, pw)),
                               dx.reshape(-1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.bwd_filter_at(x, dy, (fh, fw), iw, (sh, sw), (ph, pw)),
                               dw.reshape(-1), rtol=1e-12, atol=1e-12)


def test_thread_count_does_not_change_results(monkeypatch):
    """Each output is summed by one thread in a fixed order."""
    s = Shape(3, 12, 12, 8, 5, 5, 1, 1, 2, 2)
    inp = make_inputs(s, "f32", seed=2)
    a = oracle.bwd_filter(inp.x.values, inp.dy.values, (5, 5), 1, 2)
    b = oracle.bwd_filter(inp.x.values, inp.dy.values, (5, 5), 1, 2)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------- planted mistakes -------

MUTATIONS = {
    # forward reads the filter turned by 180 degrees (a true convolution)
    "fwd_flipped_filter": ("dwc_oracle_fwd(", "WAT(&d, w, kh, kw, 0)",
                           "WAT(&d, w, d.fh - 1 - kh, d.fw - 1 - kw, 0)"),
    # forward padding off by one row
    "fwd_pad_off_by_one": ("dwc_oracle_fwd(", "int64_t h = oh * d.sh - d.ph + kh;",
                           "int64_t h = oh * d.sh - d.ph + kh + 1;"),
    # forward drops the last tap of every filter row
    "fwd_dropped_tap": ("dwc_oracle_fwd(", "kw < d.fw; ++kw", "kw < d.fw - 1; ++kw"),
    # forward ignores the stride along the width
    "fwd_width_stride": ("dwc_oracle_fwd(", "ow * d.sw - d.pw + kw", "ow - d.pw + kw"),
    # data gradient with a sign error
    "bwd_data_sign": ("dwc_oracle_bwd_data(", "xp[cc] += gp[cc] * wp[cc]",
                      "xp[cc] -= gp[cc] * wp[cc]"),
    # data gradient scattering with the unflipped tap (transposed operand)
    "bwd_data_transposed_tap": ("dwc_oracle_bwd_data(", "WAT(&d, w, kh, kw, 0)",
                                "WAT(&d, w, d.fh - 1 - kh, d.fw - 1 - kw, 0)"),
    # filter gradient with rows and columns of the tap swapped
    "bwd_filter_swapped_tap": ("dwc_oracle_bwd_filter(", "double* ap = &acc[kw * d.c];",
                               "double* ap = &acc[(d.fw - 1 - kw) * d.c];"),
    # filter gradient that forgets the padding offset along the width
    "bwd_filter_no_pad": ("dwc_oracle_bwd_filter(", "ow * d.sw - d.pw + kw",
                          "ow * d.sw + kw"),
}


def _mutant(tmp_path, name):
    func, old, new = MUTATIONS[name]
    src = open(oracle.SRC).read()
    start = src.index("int " + func)
    nxt = src.find("\nint dwc_oracle_", start + 1)
    end = len(src) if nxt < 0 else nxt
    body = src[start:end]
    assert old in body, (name, old)
    mutated = src[:start] + body.replace(old, new) + src[end:]
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    so = str(tmp_path / f"lib_{name}.so")
    oracle.compile_c(str(path), so)
    return oracle.Oracle(so)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    """The golden examples fail for every planted mistake (they are 3x3
    images, square, so no mutant can index outside its buffers)."""
    bad = _mutant(tmp_path, name)
    with pytest.raises(AssertionError):
        check_golden(bad)

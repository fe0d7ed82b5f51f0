"""Pins of the oracle's fused prologue (Flash-DWC §5.2: batch normalisation
and activation applied to X before the forward), each against something other
than the oracle's own formula."""

import math

import numpy as np
import pytest

import oracle


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_activation_values_by_hand():
    t = np.array([-7.0, -1.0, 0.0, 1.0, 2.5, 7.0])
    assert np.array_equal(oracle.activation(t, "none"), t)
    assert np.array_equal(oracle.activation(t, "relu"), [0, 0, 0, 1, 2.5, 7])
    assert np.array_equal(oracle.activation(t, "relu6"), [0, 0, 0, 1, 2.5, 6])
    # silu(1) = 1 / (1 + 1/e); silu(-1) = -1 / (1 + e); silu(0) = 0
    s = oracle.activation(np.array([1.0, -1.0, 0.0, 40.0, -800.0]), "silu")
    assert s[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert s[1] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert s[2] == 0.0
    assert s[3] == pytest.approx(40.0, rel=1e-15)  # t * sigmoid(t) -> t
    assert s[4] == 0.0  # -> 0 from below
    with pytest.raises(ValueError):
        oracle.activation(t, "gelu")


def test_identity_prologue_is_the_plain_forward():
    r = _rng(1)
    x = r.standard_normal((2, 7, 8, 5))
    w = r.standard_normal((3, 5, 5))
    y = oracle.fwd_fused(x, np.ones(5), np.zeros(5), "none", w, 1, (1, 2))
    assert np.array_equal(y, oracle.fwd(x, w, 1, (1, 2)))


def test_prologue_is_per_channel():
    r = _rng(2)
    x = r.standard_normal((1, 3, 4, 6))
    scale, shift = r.standard_normal(6), r.standard_normal(6)
    xp = oracle.prologue(x, scale, shift, "relu")
    for c in range(6):
        assert np.array_equal(xp[..., c], np.maximum(x[..., c] * scale[c] + shift[c], 0.0))


def test_relu_below_zero_gives_zero_output():
    r = _rng(3)
    x = r.uniform(-1, 1, (2, 6, 6, 4))
    w = r.standard_normal((3, 3, 4))
    y = oracle.fwd_fused(x, np.full(4, 0.5), np.full(4, -1.0), "relu", w, 1, 1)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("act", ["relu", "relu6", "silu"])
def test_constant_input_closed_form_keeps_padding_zero(act):
    """X = 1: X' = act(scale + shift) everywhere inside the image and the
    padding stays 0, so an output sums the filter taps that land inside the
    image times that constant -- at the corner, the taps of the lower-right
    part only."""
    c = 3
    scale, shift = np.array([2.0, -0.5, 1.5]), np.array([0.5, -1.0, 5.0])
    w = _rng(4).standard_normal((3, 3, c))
    y = oracle.fwd_fused(np.ones((1, 5, 5, c)), scale, shift, act, w, 1, 1)
    k = oracle.activation(scale + shift, act)
    assert np.allclose(y[0, 2, 2], k * w.sum(axis=(0, 1)), rtol=1e-14, atol=1e-14)
    assert np.allclose(y[0, 0, 0], k * w[1:, 1:].sum(axis=(0, 1)), rtol=1e-14, atol=1e-14)
    assert np.allclose(y[0, 0, 2], k * w[1:, :].sum(axis=(0, 1)), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("act", ["none", "relu", "relu6", "silu"])
@pytest.mark.parametrize("stride", [1, 2])
def test_against_torch_functional_in_float64(act, stride):
    """An independent formulation: torch's activations and
    conv2d(groups=C) on NCHW tensors, in float64 on the CPU."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    r = _rng(5 + stride)
    n, h, wd, c, fh, fw = 2, 9, 10, 6, 5, 3
    x = r.standard_normal((n, h, wd, c)) * 3
    w = r.standard_normal((fh, fw, c))
    scale, shift = r.standard_normal(c), r.standard_normal(c)
    got = oracle.fwd_fused(x, scale, shift, act, w, stride, (2, 1))
    t = torch.from_numpy(x).permute(0, 3, 1, 2) * torch.from_numpy(scale).view(1, c, 1, 1) \
        + torch.from_numpy(shift).view(1, c, 1, 1)
    t = {"none": lambda v: v, "relu": F.relu, "relu6": F.relu6, "silu": F.silu}[act](t)
    wt = torch.from_numpy(w).permute(2, 0, 1).unsqueeze(1)
    want = F.conv2d(t, wt, stride=stride, padding=(2, 1), groups=c).permute(0, 2, 3, 1).numpy()
    assert got.shape == want.shape
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)

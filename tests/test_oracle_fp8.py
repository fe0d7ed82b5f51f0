"""Pins of the oracle's fp8 dequantisation (Flash-DWC, TACO, §7, low-bit
operands; formats: the OCP 8-bit floating-point e4m3 and e5m2 encodings).

The decoder is checked against what fixes it independently: torch's own
float8 conversion over all 256 codes, the formats' documented extreme
values and special codes, sign symmetry and ordering, and the convolution of
fp8 operands against exact integer arithmetic.
"""

import numpy as np
import pytest
import torch

import dwc_inputs
import oracle

TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
CODES = np.arange(256, dtype=np.uint8)


@pytest.mark.parametrize("fmt", oracle.FP8_FORMATS)
def test_decode_matches_torch_on_every_code(fmt):
    ours = oracle.fp8_decode(CODES, fmt)
    ref = torch.from_numpy(CODES.copy()).view(TORCH_FP8[fmt]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_documented_values():
    d = lambda c: float(oracle.fp8_decode(np.array([c], dtype=np.uint8), "e4m3")[0])
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0          # largest finite
    assert d(0x08) == 2.0 ** -6      # smallest normal
    assert d(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert d(0x01) == 2.0 ** -9      # smallest subnormal
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    v = oracle.fp8_decode(CODES, "e4m3")
    assert set(np.flatnonzero(np.isnan(v))) == {0x7F, 0xFF}
    assert not np.any(np.isinf(v))


def test_e5m2_documented_values():
    d = lambda c: float(oracle.fp8_decode(np.array([c], dtype=np.uint8), "e5m2")[0])
    assert d(0x3C) == 1.0
    assert d(0x7B) == 57344.0        # largest finite
    assert d(0x04) == 2.0 ** -14     # smallest normal
    assert d(0x01) == 2.0 ** -16     # smallest subnormal
    assert d(0x7C) == np.inf and d(0xFC) == -np.inf
    v = oracle.fp8_decode(CODES, "e5m2")
    assert set(np.flatnonzero(np.isnan(v))) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}


@pytest.mark.parametrize("fmt", oracle.FP8_FORMATS)
def test_sign_symmetry_and_order(fmt):
    v = oracle.fp8_decode(CODES, fmt)
    pos = v[:128]
    fin = np.isfinite(pos)
    assert np.all(np.diff(pos[fin]) > 0)  # codes 0 .. 0x7E (0x7B) increase
    both = np.isfinite(pos) & np.isfinite(v[128:])
    assert np.array_equal(-pos[both], v[128:][both])


@pytest.mark.parametrize("fmt", oracle.FP8_FORMATS)
def test_products_exact_in_float32(fmt):
    # the fact behind exact fp8 products in fp32 arithmetic: every product of
    # two finite values has <= 2 * (mantissa bits + 1) significant bits and
    # stays inside float32's exponent range
    v = oracle.fp8_decode(CODES, fmt)
    v = v[np.isfinite(v)]
    p = np.multiply.outer(v, v)
    assert np.array_equal(p.astype(np.float32).astype(np.float64), p)


@pytest.mark.parametrize("fmt", oracle.FP8_FORMATS)
def test_fp8_convolution_matches_integer_arithmetic(fmt):
    # small integers are exact fp8 values (|k| <= 16 in both formats): the
    # convolution of decoded codes must equal integer arithmetic exactly
    rng = np.random.default_rng(5)
    tcode = {float(x): c for c, x in enumerate(oracle.fp8_decode(CODES, fmt)) if np.isfinite(x)}
    xi = rng.integers(-4, 5, size=(2, 7, 6, 3))
    wi = rng.integers(-3, 4, size=(3, 3, 3))
    to_codes = np.vectorize(lambda k: tcode[float(k)])
    x = oracle.fp8_decode(to_codes(xi).astype(np.uint8), fmt)
    w = oracle.fp8_decode(to_codes(wi).astype(np.uint8), fmt)
    y = oracle.fwd(x, w, 1, 1)
    xp = np.pad(xi, ((0, 0), (1, 1), (1, 1), (0, 0)))
    yi = np.zeros((2, 7, 6, 3), dtype=np.int64)
    for a in range(3):
        for b in range(3):
            yi += xp[:, a:a + 7, b:b + 6, :] * wi[a, b]
    assert np.array_equal(y, yi.astype(np.float64))


@pytest.mark.parametrize("fmt", oracle.FP8_FORMATS)
def test_generated_operands_are_fp8_codes(fmt):
    s = dwc_inputs.Shape(2, 9, 9, 16, 3, 3, 1, 1, 1, 1)
    inp = dwc_inputs.make_inputs(s, fmt, seed=1)
    for op in (inp.x, inp.w, inp.dy):
        assert op.stored.dtype == np.uint8
        assert np.array_equal(oracle.fp8_decode(op.stored, fmt), op.values.astype(np.float64))

"""Helpers for the GPU parity tests: upload seeded inputs, compare with the
oracle by relative L2 error and by an elementwise error bound."""

from __future__ import annotations

import numpy as np
import torch

import depthwise_convolution_dwc_amd as dwc
from dwc_inputs import Operand

# Tolerances on max relative L2 error per tensor: fp32 operands 1e-5;
# bf16/fp16 operands with fp32 accumulation 3e-3; fp8 operands (exact
# products, fp32 outputs) the same reduced-precision budget, 3e-3 -- their
# elementwise bound (fp8 matrix-core sums) is checked separately.
TOL = {"f32": 1e-5, "bf16": 3e-3, "f16": 3e-3, "e4m3": 3e-3, "e5m2": 3e-3}
# Elementwise bound for fp8 operands: |got - want| <= FP8_EL_TOL * the same
# operation on |operands|.  The fp8 MFMAs sum each group of products with an
# error up to about 2^-12 of the sum of their magnitudes (measured on
# MI355X); the vector kernels round in fp32 (2^-24 per addition).
FP8_EL_TOL = 2.0 ** -11
# fp32 unit roundoff.
U32 = 2.0 ** -24


def gamma(k: int) -> float:
    """k*u / (1 - k*u), u = 2^-24: a sum of k terms, each a product, computed
    in fp32 in any order (any summation tree, FMA or separate rounding) is
    off by at most gamma(k+1) times the sum of the terms' magnitudes
    (the classical bound for floating-point inner products, Higham, Accuracy
    and Stability of Numerical Algorithms, chapter 3)."""
    ku = k * U32
    return ku / (1.0 - ku)


def terms_per_output(op: str, shape) -> int:
    """Most products in one output's sum: the taps of one output pixel
    (forward), the taps that land on one input pixel (data gradient: every
    stride-th tap in each direction), or every output pixel of the batch
    (filter gradient)."""
    s = shape
    if op == "fwd":
        return s.fh * s.fw
    if op == "bwd_data":
        return -(-s.fh // s.stride_h) * -(-s.fw // s.stride_w)
    return s.n * s.oh * s.ow


def el_bound(op: str, shape, dtype: str) -> float:
    """Elementwise bound, as a multiple of the same operation on |operands|:
    fp32 summation of the output's terms, plus for fp8 operands the matrix
    cores' group sums (FP8_EL_TOL)."""
    b = gamma(terms_per_output(op, shape) + 1)
    if dtype in ("e4m3", "e5m2"):
        b += FP8_EL_TOL
    return b


def check_parity(got, want, mag, op: str, shape, dtype: str, what=""):
    """Asserts relative L2 <= TOL[dtype] over the whole tensor and
    |got - want| <= el_bound * mag for every element, where mag is the same
    operation on |operands| (so the bound scales with each output's own
    terms).  Returns (rel_l2, worst |got - want| / (el_bound * mag))."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert got.shape == want.shape == mag.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = rel_l2(got, want)
    assert err <= TOL[dtype], f"{what}: rel_l2 {err:.3e} > {TOL[dtype]}"
    lim = el_bound(op, shape, dtype) * mag + 1e-300
    d = np.abs(got - want)
    worst = float(np.max(d / lim)) if d.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(d / lim)), d.shape)
        raise AssertionError(f"{what}: elementwise bound broken at {i}: got {got[i]!r} "
                             f"want {want[i]!r} bound {lim[i]:.3e} ({worst:.3g}x)")
    return err, worst


def to_device(op: Operand, device="cuda") -> torch.Tensor:
    if op.dtype == "f32":
        return torch.from_numpy(op.stored).to(device)
    if op.dtype == "f16":
        return torch.from_numpy(op.stored).to(device)
    if op.dtype in ("e4m3", "e5m2"):
        tdt = torch.float8_e4m3fn if op.dtype == "e4m3" else torch.float8_e5m2
        return torch.from_numpy(op.stored).to(device).view(tdt)
    # bf16 bits travel as int16 and are reinterpreted on the device
    return torch.from_numpy(op.stored.view(np.int16)).to(device).view(torch.bfloat16)


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    want = np.asarray(want, dtype=np.float64).reshape(-1)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return float(num)
    return float(num / den)


def sample_index(shape, k, rng) -> np.ndarray:
    """k random multi-indices into ``shape`` (rows of an int64 array), always
    including the first and last element."""
    k = min(k, int(np.prod(shape)))
    idx = np.stack([rng.integers(0, s, size=k) for s in shape], axis=1)
    idx[0] = 0
    idx[-1] = np.asarray(shape) - 1
    return idx.astype(np.int64)


def gather(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    it = torch.from_numpy(idx).to(t.device)
    return t[tuple(it[:, d] for d in range(idx.shape[1]))].double().cpu().numpy()


def sync():
    torch.cuda.synchronize()


def log(*a):
    print(*a, flush=True)


__all__ = ["TOL", "FP8_EL_TOL", "U32", "gamma", "terms_per_output", "el_bound", "check_parity",
           "to_device", "rel_l2", "sample_index", "gather", "sync", "log", "dwc"]

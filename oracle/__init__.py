"""CPU oracle for depthwise convolution -- TEST INFRASTRUCTURE ONLY.

The oracle is the plain float64 direct-loop definition of DWC forward, data
gradient and filter gradient (Flash-DWC, TACO: §2.1 for the per-channel inner
product, §2.3 for the channel-last layouts, §5.1 for the two backward
operators).  The arithmetic lives in ``dwc_oracle.c``; this module builds it
with gcc and calls it through ctypes.  The fused prologue of §5.2 (per-channel
scale and shift, then an activation, applied to X before the forward) is an
elementwise float64 map written here in numpy.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does, and the two share no code.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dwc_oracle.c")
LIB = os.path.join(HERE, "libdwc_oracle.so")

_I64 = ctypes.c_int64
_PD = ctypes.POINTER(ctypes.c_double)
_PI = ctypes.POINTER(ctypes.c_int64)


def compile_c(src: str, out: str) -> str:
    """gcc -O2 with OpenMP and without fast-math: sums keep IEEE semantics."""
    tmp = out + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
         "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        compile_c(SRC, LIB)
    return LIB


def _f64(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_PD)


def _pair(v) -> Tuple[int, int]:
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _dims(n, h, w, c, fh, fw, stride, pad):
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    return [n, h, w, c, fh, fw, sh, sw, ph, pw]


def _idx(idx: np.ndarray, width: int) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert idx.ndim == 2 and idx.shape[1] == width
    return idx


class Oracle:
    """One compiled copy of the oracle (the real one, or a planted-mistake
    copy in the mutation tests)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dims = [_I64] * 10
        for name in ("dwc_oracle_fwd", "dwc_oracle_bwd_data", "dwc_oracle_bwd_filter"):
            f = getattr(lib, name)
            f.argtypes = dims + [_PD, _PD, _PD]
            f.restype = ctypes.c_int
        for name in ("dwc_oracle_fwd_at", "dwc_oracle_bwd_data_at",
                     "dwc_oracle_bwd_filter_at"):
            f = getattr(lib, name)
            f.argtypes = dims + [_PD, _PD, _PI, _I64, _PD]
            f.restype = ctypes.c_int
        lib.dwc_oracle_output_dims.argtypes = [_I64] * 8 + [_PI, _PI]
        lib.dwc_oracle_output_dims.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def output_dims(self, h, w, fh, fw, stride=1, pad=0) -> Tuple[int, int]:
        sh, sw = _pair(stride)
        ph, pw = _pair(pad)
        oh, ow = _I64(), _I64()
        rc = self.lib.dwc_oracle_output_dims(h, w, fh, fw, sh, sw, ph, pw,
                                             ctypes.byref(oh), ctypes.byref(ow))
        if rc:
            raise ValueError("bad convolution geometry")
        return oh.value, ow.value

    def fwd(self, x: np.ndarray, w: np.ndarray, stride=1, pad=0) -> np.ndarray:
        """Y = DWC(X, W): x is N x H x W x C, w is FH x FW x C."""
        x, w = _f64(x), _f64(w)
        n, h, wd, c = x.shape
        fh, fw, c2 = w.shape
        assert c == c2
        oh, ow = self.output_dims(h, wd, fh, fw, stride, pad)
        y = np.empty((n, oh, ow, c), dtype=np.float64)
        rc = self.lib.dwc_oracle_fwd(*_dims(n, h, wd, c, fh, fw, stride, pad),
                                     _p(x), _p(w), _p(y))
        if rc:
            raise ValueError("oracle fwd: bad arguments")
        return y

    def bwd_data(self, dy: np.ndarray, w: np.ndarray, in_hw: Sequence[int],
                 stride=1, pad=0) -> np.ndarray:
        """dX for input spatial size ``in_hw`` (several H can give one OH)."""
        dy, w = _f64(dy), _f64(w)
        n, oh, ow, c = dy.shape
        fh, fw, c2 = w.shape
        assert c == c2
        h, wd = int(in_hw[0]), int(in_hw[1])
        assert self.output_dims(h, wd, fh, fw, stride, pad) == (oh, ow)
        dx = np.empty((n, h, wd, c), dtype=np.float64)
        rc = self.lib.dwc_oracle_bwd_data(*_dims(n, h, wd, c, fh, fw, stride, pad),
                                          _p(dy), _p(w), _p(dx))
        if rc:
            raise ValueError("oracle bwd_data: bad arguments")
        return dx

    def bwd_filter(self, x: np.ndarray, dy: np.ndarray, f_hw: Sequence[int],
                   stride=1, pad=0) -> np.ndarray:
        """dW (FH x FW x C) from X and dY."""
        x, dy = _f64(x), _f64(dy)
        n, h, wd, c = x.shape
        fh, fw = int(f_hw[0]), int(f_hw[1])
        assert self.output_dims(h, wd, fh, fw, stride, pad) == tuple(dy.shape[1:3])
        dw = np.empty((fh, fw, c), dtype=np.float64)
        rc = self.lib.dwc_oracle_bwd_filter(*_dims(n, h, wd, c, fh, fw, stride, pad),
                                            _p(x), _p(dy), _p(dw))
        if rc:
            raise ValueError("oracle bwd_filter: bad arguments")
        return dw

    def fwd_at(self, x, w, idx, stride=1, pad=0) -> np.ndarray:
        """Y at the (n, oh, ow, c) rows of ``idx``."""
        x, w = _f64(x), _f64(w)
        idx = _idx(idx, 4)
        n, h, wd, c = x.shape
        fh, fw, _ = w.shape
        out = np.empty(len(idx), dtype=np.float64)
        rc = self.lib.dwc_oracle_fwd_at(*_dims(n, h, wd, c, fh, fw, stride, pad), _p(x), _p(w),
                                        idx.ctypes.data_as(_PI), len(idx), _p(out))
        if rc:
            raise ValueError("oracle fwd_at: bad arguments")
        return out

    def bwd_data_at(self, dy, w, in_hw, idx, stride=1, pad=0) -> np.ndarray:
        """dX at the (n, ih, iw, c) rows of ``idx``."""
        dy, w = _f64(dy), _f64(w)
        idx = _idx(idx, 4)
        n, _, _, c = dy.shape
        fh, fw, _ = w.shape
        h, wd = int(in_hw[0]), int(in_hw[1])
        out = np.empty(len(idx), dtype=np.float64)
        rc = self.lib.dwc_oracle_bwd_data_at(*_dims(n, h, wd, c, fh, fw, stride, pad),
                                             _p(dy), _p(w), idx.ctypes.data_as(_PI),
                                             len(idx), _p(out))
        if rc:
            raise ValueError("oracle bwd_data_at: bad arguments")
        return out

    def bwd_filter_at(self, x, dy, f_hw, idx, stride=1, pad=0) -> np.ndarray:
        """dW at the (fh, fw, c) rows of ``idx``."""
        x, dy = _f64(x), _f64(dy)
        idx = _idx(idx, 3)
        n, h, wd, c = x.shape
        fh, fw = int(f_hw[0]), int(f_hw[1])
        out = np.empty(len(idx), dtype=np.float64)
        rc = self.lib.dwc_oracle_bwd_filter_at(*_dims(n, h, wd, c, fh, fw, stride, pad),
                                               _p(x), _p(dy), idx.ctypes.data_as(_PI),
                                               len(idx), _p(out))
        if rc:
            raise ValueError("oracle bwd_filter_at: bad arguments")
        return out


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default


def output_dims(*a, **k):
    return get().output_dims(*a, **k)


def fwd(*a, **k):
    return get().fwd(*a, **k)


def bwd_data(*a, **k):
    return get().bwd_data(*a, **k)


def bwd_filter(*a, **k):
    return get().bwd_filter(*a, **k)


def fwd_at(*a, **k):
    return get().fwd_at(*a, **k)


def bwd_data_at(*a, **k):
    return get().bwd_data_at(*a, **k)


def bwd_filter_at(*a, **k):
    return get().bwd_filter_at(*a, **k)


# --------------------------------------------------------------------------
# Fused prologue (Flash-DWC, TACO, §5.2 "kernel fusion": the batch
# normalisation and activation that usually precede a DWC, applied to X as
# part of the forward).  Read as inference-form batch normalisation -- one
# scale and shift per channel -- followed by the activation, in float64.
# --------------------------------------------------------------------------

ACTIVATIONS = ("none", "relu", "relu6", "silu")


def activation(t: np.ndarray, act: str) -> np.ndarray:
    """none: t; relu: max(t, 0); relu6: min(max(t, 0), 6);
    silu: t * sigmoid(t) = t / (1 + exp(-t))."""
    t = _f64(t)
    if act == "none":
        return t
    if act == "relu":
        return np.maximum(t, 0.0)
    if act == "relu6":
        return np.minimum(np.maximum(t, 0.0), 6.0)
    if act == "silu":
        with np.errstate(over="ignore"):
            return t / (1.0 + np.exp(-t))
    raise ValueError(f"unknown activation {act!r}")


def prologue(x: np.ndarray, scale: np.ndarray, shift: np.ndarray, act: str) -> np.ndarray:
    """X'[n, h, w, c] = act(X[n, h, w, c] * scale[c] + shift[c])."""
    return activation(_f64(x) * _f64(scale) + _f64(shift), act)


def fwd_fused(x, scale, shift, act, w, stride=1, pad=0) -> np.ndarray:
    """Forward DWC of the prologue's output; the zero padding surrounds X'
    (padding positions are zero after the prologue, not act(shift))."""
    return fwd(prologue(x, scale, shift, act), w, stride, pad)


# --------------------------------------------------------------------------
# Low-bit operands (Flash-DWC, TACO, §7 "scalability", low-bit data types:
# operands stored and multiplied in 8 bits, sums kept in higher precision).
# The pages name FP8 without fixing an encoding; read here as the two OCP
# 8-bit floating-point formats that CDNA4 matrix cores take:
#   e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
#         is subnormal (m / 8 * 2^-6); S.1111.111 is NaN; no infinities, so
#         exponent field 15 with mantissa 0..6 are ordinary numbers (max 448);
#   e5m2: sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-754 style:
#         exponent field 0 is subnormal (m / 4 * 2^-14), 31 is +-inf (m = 0)
#         or NaN (m != 0); max 57344.
# Dequantisation is exact in float64, so the convolution of fp8 operands is
# the float64 oracle applied to the decoded values.
# --------------------------------------------------------------------------

FP8_FORMATS = ("e4m3", "e5m2")
_FP8_LAYOUT = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}  # exponent bits, mantissa bits, bias


def fp8_decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """float64 values of fp8 codes (uint8) in format fmt (``FP8_FORMATS``)."""
    if fmt not in _FP8_LAYOUT:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    eb, mb, bias = _FP8_LAYOUT[fmt]
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = (c & ((1 << mb) - 1)).astype(np.float64)
    frac = m / float(1 << mb)
    mag = np.where(e == 0, np.ldexp(frac, 1 - bias), np.ldexp(1.0 + frac, e - bias))
    top = (1 << eb) - 1
    if fmt == "e4m3":
        mag = np.where((e == top) & ((c & 7) == 7), np.nan, mag)
    else:
        mag = np.where(e == top, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag

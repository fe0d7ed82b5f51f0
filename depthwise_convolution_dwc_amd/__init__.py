"""Python binding of libdwc, depthwise convolution for MI355X (gfx950).

Argument marshalling only: every operation runs in the HIP kernels of
``libdwc.so`` (built from ``csrc/`` by ``build.py``), called through its C
ABI (``include/dwc.h``).  PyTorch supplies device memory and the current
stream.  If the library has not been built, every call raises: there is no
fallback.

Operations (Flash-DWC: Making Depthwise Convolution Compute-Efficient on
GPUs, TACO): ``fwd`` is the forward DWC of §2.1, ``bwd_data`` and
``bwd_filter`` are the data and filter gradients of §5.1.  Tensors are
channel-last (§2.3): X, Y as N x H x W x C, the filter as FH x FW x C.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch  # loaded first: libdwc then binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdwc.so")

F32, BF16, F16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
ALGO = {"auto": 0, "vector": 1, "direct": 1, "mfma": 2, "generic": 3, "hybrid": 4}
ACT = {"none": 0, "relu": 1, "relu6": 2, "silu": 3}
OP_FWD, OP_BWD_DATA, OP_BWD_FILTER = 0, 1, 2
# DWC_NOALLOC_SCRATCH_BYTES: the fixed scratch of dwc_bwd_filter_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20

_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16,
               torch.float8_e4m3fn: FP8_E4M3, torch.float8_e5m2: FP8_E5M2}

EXPORTED = (
    "dwc_version", "dwc_status_string", "dwc_last_error", "dwc_output_dims",
    "dwc_check", "dwc_plan_describe", "dwc_fwd", "dwc_fwd_fused", "dwc_bwd_data",
    "dwc_bwd_filter_workspace_size", "dwc_bwd_filter", "dwc_bwd_filter_noalloc",
)


class Problem(ctypes.Structure):
    """Mirror of ``dwc_problem`` in include/dwc.h."""

    _fields_ = [
        ("n", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
        ("c", ctypes.c_int64),
        ("fh", ctypes.c_int32), ("fw", ctypes.c_int32),
        ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
        ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("algo", ctypes.c_int32), ("wgrad_split", ctypes.c_int32),
    ]


class DwcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libdwc error {status}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libdwc.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m depthwise_convolution_dwc_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
        l.dwc_version.restype = ctypes.c_int
        l.dwc_status_string.argtypes = [ctypes.c_int]
        l.dwc_status_string.restype = ctypes.c_char_p
        l.dwc_last_error.restype = ctypes.c_char_p
        l.dwc_output_dims.argtypes = [P, i64p, i64p]
        l.dwc_check.argtypes = [P, ctypes.c_int]
        l.dwc_plan_describe.argtypes = [P, ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t]
        l.dwc_fwd.argtypes = [P, vp, vp, vp, vp]
        l.dwc_fwd_fused.argtypes = [P, vp, vp, vp, ctypes.c_int, vp, vp, vp]
        l.dwc_bwd_data.argtypes = [P, vp, vp, vp, vp]
        l.dwc_bwd_filter_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        l.dwc_bwd_filter.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        l.dwc_bwd_filter_noalloc.argtypes = [P, vp, vp, vp, vp]
        for name in EXPORTED:
            if name not in ("dwc_status_string", "dwc_last_error"):
                getattr(l, name).restype = ctypes.c_int
        _lib = l
    return _lib


def _raise(status: int):
    if status != 0:
        raise DwcError(status, lib().dwc_last_error().decode())


def _pair(v) -> Tuple[int, int]:
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def problem(n, h, w, c, fh, fw, stride=1, pad=0, dtype=F32, algo="auto",
            wgrad_split=0) -> Problem:
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPE_CODE[dtype]
    return Problem(n, h, w, c, fh, fw, sh, sw, ph, pw, dtype, F32,
                   ALGO[algo] if isinstance(algo, str) else int(algo), wgrad_split)


def output_dims(p: Problem) -> Tuple[int, int]:
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    _raise(lib().dwc_output_dims(ctypes.byref(p), ctypes.byref(oh), ctypes.byref(ow)))
    return oh.value, ow.value


def check(p: Problem, op: int) -> int:
    return lib().dwc_check(ctypes.byref(p), op)


def plan_describe(p: Problem, op: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _raise(lib().dwc_plan_describe(ctypes.byref(p), op, buf, len(buf)))
    return buf.value.decode()


def workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t()
    _raise(lib().dwc_bwd_filter_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def last_error() -> str:
    return lib().dwc_last_error().decode()


# --------------------------------------------------------------------------
# Raw-pointer calls (device addresses as ints; stream as an int handle).
# --------------------------------------------------------------------------

def fwd_ptr(p: Problem, x: int, w: int, y: int, stream: int = 0) -> None:
    _raise(lib().dwc_fwd(ctypes.byref(p), x, w, y, stream))


def fwd_fused_ptr(p: Problem, x: int, scale: int, shift: int, act: int, w: int, y: int,
                  stream: int = 0) -> None:
    _raise(lib().dwc_fwd_fused(ctypes.byref(p), x, scale, shift, act, w, y, stream))


def bwd_data_ptr(p: Problem, dy: int, w: int, dx: int, stream: int = 0) -> None:
    _raise(lib().dwc_bwd_data(ctypes.byref(p), dy, w, dx, stream))


def bwd_filter_ptr(p: Problem, x: int, dy: int, dw: int, ws: int, ws_bytes: int,
                   stream: int = 0) -> None:
    _raise(lib().dwc_bwd_filter(ctypes.byref(p), x, dy, dw, ws, ws_bytes, stream))


def bwd_filter_noalloc_ptr(p: Problem, x: int, dy: int, dw: int, stream: int = 0) -> None:
    _raise(lib().dwc_bwd_filter_noalloc(ctypes.byref(p), x, dy, dw, stream))


# --------------------------------------------------------------------------
# Tensor calls.
# --------------------------------------------------------------------------

def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_tensor(t: torch.Tensor, name: str, ndim: int, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (channel-last), got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (N x H x W x C / FH x FW x C)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _operand_dtype(*ts: torch.Tensor) -> int:
    dts = {t.dtype for t in ts}
    if len(dts) != 1 or next(iter(dts)) not in _DTYPE_CODE:
        raise TypeError("operands must share one of float32/bfloat16/float16/"
                        f"float8_e4m3fn/float8_e5m2, got {dts}")
    return _DTYPE_CODE[ts[0].dtype]


def fwd(x: torch.Tensor, w: torch.Tensor, stride=1, pad=0, out: Optional[torch.Tensor] = None,
        algo="auto", stream=None) -> torch.Tensor:
    """Y = DWC(X, W); x: N x H x W x C, w: FH x FW x C; Y is fp32."""
    _check_tensor(x, "x", 4)
    _check_tensor(w, "w", 3)
    dt = _operand_dtype(x, w)
    n, h, wd, c = x.shape
    fh, fw, c2 = w.shape
    if c2 != c:
        raise ValueError("x and w disagree on C")
    p = problem(n, h, wd, c, fh, fw, stride, pad, dt, algo)
    oh, ow = output_dims(p)
    if out is None:
        out = torch.empty((n, oh, ow, c), dtype=torch.float32, device=x.device)
    _check_tensor(out, "out", 4, torch.float32)
    if tuple(out.shape) != (n, oh, ow, c):
        raise ValueError(f"out must be {(n, oh, ow, c)}")
    fwd_ptr(p, x.data_ptr(), w.data_ptr(), out.data_ptr(), _stream(stream))
    return out


def fwd_fused(x: torch.Tensor, w: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
              act: str = "relu", stride=1, pad=0, out: Optional[torch.Tensor] = None,
              algo="auto", stream=None) -> torch.Tensor:
    """Y = DWC(act(X * scale + shift), W) with the prologue fused into the
    forward (scale, shift: C fp32 values); Y is fp32."""
    _check_tensor(x, "x", 4)
    _check_tensor(w, "w", 3)
    _check_tensor(scale, "scale", 1, torch.float32)
    _check_tensor(shift, "shift", 1, torch.float32)
    dt = _operand_dtype(x, w)
    n, h, wd, c = x.shape
    fh, fw, c2 = w.shape
    if c2 != c or scale.shape[0] != c or shift.shape[0] != c:
        raise ValueError("x, w, scale and shift disagree on C")
    if act not in ACT:
        raise ValueError(f"act must be one of {sorted(ACT)}")
    p = problem(n, h, wd, c, fh, fw, stride, pad, dt, algo)
    oh, ow = output_dims(p)
    if out is None:
        out = torch.empty((n, oh, ow, c), dtype=torch.float32, device=x.device)
    _check_tensor(out, "out", 4, torch.float32)
    if tuple(out.shape) != (n, oh, ow, c):
        raise ValueError(f"out must be {(n, oh, ow, c)}")
    fwd_fused_ptr(p, x.data_ptr(), scale.data_ptr(), shift.data_ptr(), ACT[act], w.data_ptr(),
                  out.data_ptr(), _stream(stream))
    return out


def bwd_data(dy: torch.Tensor, w: torch.Tensor, in_hw: Sequence[int], stride=1, pad=0,
             out: Optional[torch.Tensor] = None, algo="auto", stream=None) -> torch.Tensor:
    """dX (N x H x W x C, fp32) for input size ``in_hw`` from dY and W."""
    _check_tensor(dy, "dy", 4)
    _check_tensor(w, "w", 3)
    dt = _operand_dtype(dy, w)
    n, oh, ow, c = dy.shape
    fh, fw, c2 = w.shape
    if c2 != c:
        raise ValueError("dy and w disagree on C")
    h, wd = int(in_hw[0]), int(in_hw[1])
    p = problem(n, h, wd, c, fh, fw, stride, pad, dt, algo)
    if output_dims(p) != (oh, ow):
        raise ValueError(f"dy spatial size {(oh, ow)} does not match input {(h, wd)}")
    if out is None:
        out = torch.empty((n, h, wd, c), dtype=torch.float32, device=dy.device)
    _check_tensor(out, "out", 4, torch.float32)
    if tuple(out.shape) != (n, h, wd, c):
        raise ValueError(f"out must be {(n, h, wd, c)}")
    bwd_data_ptr(p, dy.data_ptr(), w.data_ptr(), out.data_ptr(), _stream(stream))
    return out


def bwd_filter(x: torch.Tensor, dy: torch.Tensor, f_hw: Sequence[int], stride=1, pad=0,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               wgrad_split: int = 0, algo="auto", stream=None) -> torch.Tensor:
    """dW (FH x FW x C, fp32) from X and dY."""
    _check_tensor(x, "x", 4)
    _check_tensor(dy, "dy", 4)
    dt = _operand_dtype(x, dy)
    n, h, wd, c = x.shape
    fh, fw = int(f_hw[0]), int(f_hw[1])
    p = problem(n, h, wd, c, fh, fw, stride, pad, dt, algo, wgrad_split)
    oh, ow = output_dims(p)
    if tuple(dy.shape) != (n, oh, ow, c):
        raise ValueError(f"dy must be {(n, oh, ow, c)}")
    if out is None:
        out = torch.empty((fh, fw, c), dtype=torch.float32, device=x.device)
    _check_tensor(out, "out", 3, torch.float32)
    if tuple(out.shape) != (fh, fw, c):
        raise ValueError(f"out must be {(fh, fw, c)}")
    need = workspace_size(p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    bwd_filter_ptr(p, x.data_ptr(), dy.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes,
                   _stream(stream))
    return out


def bwd_filter_noalloc(x: torch.Tensor, dy: torch.Tensor, f_hw: Sequence[int], stride=1, pad=0,
                       out: torch.Tensor = None, wgrad_split: int = 0, algo="auto",
                       stream=None) -> torch.Tensor:
    """dW (FH x FW x C, fp32) from X and dY through the entry point that
    allocates nothing: the slice partials live in the library's fixed
    per-device scratch.  ``out`` must be given (this call allocates no
    device memory, torch's included)."""
    _check_tensor(x, "x", 4)
    _check_tensor(dy, "dy", 4)
    dt = _operand_dtype(x, dy)
    n, h, wd, c = x.shape
    fh, fw = int(f_hw[0]), int(f_hw[1])
    p = problem(n, h, wd, c, fh, fw, stride, pad, dt, algo, wgrad_split)
    oh, ow = output_dims(p)
    if tuple(dy.shape) != (n, oh, ow, c):
        raise ValueError(f"dy must be {(n, oh, ow, c)}")
    if out is None:
        raise ValueError("out must be given: bwd_filter_noalloc allocates nothing")
    _check_tensor(out, "out", 3, torch.float32)
    if tuple(out.shape) != (fh, fw, c):
        raise ValueError(f"out must be {(fh, fw, c)}")
    bwd_filter_noalloc_ptr(p, x.data_ptr(), dy.data_ptr(), out.data_ptr(), _stream(stream))
    return out

"""PyTorch autograd wrapper of libdwc: a depthwise Conv2d whose forward,
data gradient and filter gradient all run in libdwc's HIP kernels.

Layouts follow the library (Flash-DWC, TACO, §2.3: channel-last tensors):
activations N x H x W x C and the filter FH x FW x C.  A module stores its
weight in that FH x FW x C layout, so a training step moves no weights
around; ``weight_from_torch`` / ``weight_to_torch`` convert from / to the
C x 1 x FH x FW layout of ``torch.nn.Conv2d(groups=C)``.

Inputs may be given channel-last (``layout="nhwc"``, a contiguous
N x H x W x C tensor) or as logical NCHW tensors in ``torch.channels_last``
memory format (``layout="nchw"``), whose memory already is N x H x W x C:
both are passed to the library without a copy.  A logical NCHW tensor in
another memory format is made channels_last first (one copy).

Outputs and gradients are computed in fp32 (the library's output type).  For
bf16/fp16 operands the forward returns fp32; the backward rounds the
incoming gradient to the operand dtype (the library takes X, W and dY in one
dtype) and returns dX and dW in the dtypes of X and W.
"""

from __future__ import annotations

import math
from typing import Tuple, Union

import torch

from . import bwd_data, bwd_filter, fwd

IntPair = Union[int, Tuple[int, int]]


def _pair(v: IntPair) -> Tuple[int, int]:
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def weight_from_torch(w: torch.Tensor) -> torch.Tensor:
    """C x 1 x FH x FW (torch.nn.Conv2d, groups = C) -> FH x FW x C, contiguous."""
    if w.dim() != 4 or w.shape[1] != 1:
        raise ValueError(f"expected a C x 1 x FH x FW depthwise weight, got {tuple(w.shape)}")
    return w[:, 0].permute(1, 2, 0).contiguous()


def weight_to_torch(w: torch.Tensor) -> torch.Tensor:
    """FH x FW x C -> C x 1 x FH x FW (torch.nn.Conv2d, groups = C), contiguous."""
    if w.dim() != 3:
        raise ValueError(f"expected an FH x FW x C weight, got {tuple(w.shape)}")
    return w.permute(2, 0, 1).unsqueeze(1).contiguous()


def _to_nhwc(x: torch.Tensor, layout: str) -> torch.Tensor:
    if layout == "nhwc":
        return x.contiguous()
    if layout == "nchw":
        if x.dim() != 4:
            raise ValueError(f"expected a 4-d NCHW tensor, got {tuple(x.shape)}")
        return x.contiguous(memory_format=torch.channels_last).permute(0, 2, 3, 1)
    raise ValueError(f"layout must be 'nhwc' or 'nchw', got {layout!r}")


def _from_nhwc(y: torch.Tensor, layout: str) -> torch.Tensor:
    # an N x H x W x C tensor seen as logical NCHW in channels_last memory
    return y if layout == "nhwc" else y.permute(0, 3, 1, 2)


class DepthwiseConv2dFunction(torch.autograd.Function):
    """Y = DWC(X, W) on channel-last tensors (X: N x H x W x C, W: FH x FW x C).

    forward: ``dwc_fwd``; backward: ``dwc_bwd_data`` for dX and
    ``dwc_bwd_filter`` for dW (Flash-DWC §5.1), at any stride and padding."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, stride: Tuple[int, int],
                pad: Tuple[int, int], algo: str) -> torch.Tensor:
        ctx.save_for_backward(x, w)
        ctx.stride, ctx.pad, ctx.algo = stride, pad, algo
        return fwd(x, w, stride, pad, algo=algo)

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        x, w = ctx.saved_tensors
        gy = gy.to(x.dtype).contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = bwd_data(gy, w, (x.shape[1], x.shape[2]), ctx.stride, ctx.pad, algo=ctx.algo)
            dx = dx.to(x.dtype)
        if ctx.needs_input_grad[1]:
            dw = bwd_filter(x, gy, (w.shape[0], w.shape[1]), ctx.stride, ctx.pad, algo=ctx.algo)
            dw = dw.to(w.dtype)
        return dx, dw, None, None, None


def depthwise_conv2d(x: torch.Tensor, weight: torch.Tensor, stride: IntPair = 1,
                     padding: IntPair = 0, layout: str = "nhwc",
                     algo: str = "auto") -> torch.Tensor:
    """Depthwise 2-D cross-correlation with autograd.

    x: N x H x W x C (``layout="nhwc"``) or logical N x C x H x W
    (``layout="nchw"``); weight: FH x FW x C.  Returns fp32 in the same
    layout as x."""
    if weight.dim() != 3:
        raise ValueError(f"weight must be FH x FW x C, got {tuple(weight.shape)}")
    xn = _to_nhwc(x, layout)
    y = DepthwiseConv2dFunction.apply(xn, weight.contiguous(), _pair(stride), _pair(padding),
                                      algo)
    return _from_nhwc(y, layout)


class DepthwiseConv2d(torch.nn.Module):
    """Depthwise Conv2d (groups = channels, no bias) on libdwc.

    The weight parameter is FH x FW x C.  Initialised like torch.nn.Conv2d:
    uniform in +-1/sqrt(FH * FW) (kaiming-uniform with a = sqrt(5) for a
    fan-in of FH * FW)."""

    def __init__(self, channels: int, kernel_size: IntPair, stride: IntPair = 1,
                 padding: IntPair = 0, layout: str = "nchw", algo: str = "auto",
                 device=None, dtype=torch.float32):
        super().__init__()
        if layout not in ("nhwc", "nchw"):
            raise ValueError(f"layout must be 'nhwc' or 'nchw', got {layout!r}")
        self.channels = int(channels)
        self.kernel_size = _pair(kernel_size)
        self.stride = _pair(stride)
        self.padding = _pair(padding)
        self.layout = layout
        self.algo = algo
        fh, fw = self.kernel_size
        self.weight = torch.nn.Parameter(torch.empty((fh, fw, self.channels), device=device,
                                                     dtype=dtype))
        bound = 1.0 / math.sqrt(fh * fw)
        with torch.no_grad():
            self.weight.uniform_(-bound, bound)

    @classmethod
    def from_torch(cls, conv: torch.nn.Conv2d, layout: str = "nchw", algo: str = "auto"):
        """A module with the weights of a depthwise torch.nn.Conv2d (no bias,
        no dilation, zero padding given as numbers)."""
        c = conv.in_channels
        if conv.groups != c or conv.out_channels != c or conv.bias is not None:
            raise ValueError("need groups == in_channels == out_channels and no bias")
        if tuple(conv.dilation) != (1, 1) or isinstance(conv.padding, str) \
                or conv.padding_mode != "zeros":
            raise ValueError("need dilation 1 and numeric zero padding")
        m = cls(c, conv.kernel_size, conv.stride, conv.padding, layout, algo,
                device=conv.weight.device, dtype=conv.weight.dtype)
        with torch.no_grad():
            m.weight.copy_(weight_from_torch(conv.weight))
        return m

    def torch_weight(self) -> torch.Tensor:
        """The weight in torch.nn.Conv2d's C x 1 x FH x FW layout (a copy)."""
        return weight_to_torch(self.weight.detach())

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return depthwise_conv2d(x, self.weight, self.stride, self.padding, self.layout,
                                self.algo)

    def extra_repr(self) -> str:
        return (f"{self.channels}, kernel_size={self.kernel_size}, stride={self.stride}, "
                f"padding={self.padding}, layout={self.layout!r}")

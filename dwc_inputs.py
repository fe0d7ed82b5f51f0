"""Seeded synthetic inputs for depthwise convolution (DWC) workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random numbers and rounds them to the storage
precision; it holds none of the convolution arithmetic.

Layouts follow the channel-last convention of Flash-DWC (TACO), §2.3
("unified channel-last layout"): X and dY are N x H x W x C, the filter is
FH x FW x C.

Workload recipe (every shape below is synthetic, no dataset is involved):
  * generator: numpy PCG64 ``default_rng(seed)``; draw order X, W, dY;
  * draws are made in float32 and then, for half-precision workloads,
    rounded to bf16 / fp16 with round-to-nearest-even, so that the oracle and
    the GPU see bit-identical operand values;
  * "normal" distributions are N(0, var): X, dY ~ N(0, 1); the filter uses
    var = 1 / (FH * FW) (e.g. 1/49 for 7x7), read as a variance;
  * "uniform" is U(-1, 1), the distribution Flash-DWC (TACO) §4.1 and
    §6.3.2 use for their accuracy measurements.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

DTYPES = ("f32", "bf16", "f16", "e4m3", "e5m2")
FP8_DTYPES = ("e4m3", "e5m2")


@dataclasses.dataclass(frozen=True)
class Shape:
    """One DWC problem: X is n x h x w x c, the filter fh x fw x c."""

    n: int
    h: int
    w: int
    c: int
    fh: int
    fw: int
    stride_h: int = 1
    stride_w: int = 1
    pad_h: int = 0
    pad_w: int = 0

    @property
    def oh(self) -> int:
        # floor((H + 2P - F) / S) + 1; the pages print no formula, this is the
        # usual reading and matches the 14 -> 14 and 56 -> 28 shapes used here.
        return (self.h + 2 * self.pad_h - self.fh) // self.stride_h + 1

    @property
    def ow(self) -> int:
        return (self.w + 2 * self.pad_w - self.fw) // self.stride_w + 1

    def x_shape(self) -> Tuple[int, int, int, int]:
        return (self.n, self.h, self.w, self.c)

    def w_shape(self) -> Tuple[int, int, int]:
        return (self.fh, self.fw, self.c)

    def y_shape(self) -> Tuple[int, int, int, int]:
        return (self.n, self.oh, self.ow, self.c)


@dataclasses.dataclass
class Operand:
    """A tensor in two forms: exact float32 values and the stored bits.

    ``values`` holds the operand as float32 (bf16/fp16/fp8 values are exactly
    representable in float32, so converting them to float64 for the oracle is
    exact).  ``stored`` is what goes to the device: float32, float16, the
    raw bf16 bit patterns as uint16, or the fp8 codes as uint8.
    """

    values: np.ndarray
    stored: np.ndarray
    dtype: str


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_operand(x32: np.ndarray, dtype: str) -> Operand:
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return Operand(values=x32, stored=x32, dtype=dtype)
    if dtype == "bf16":
        bits = round_to_bf16_bits(x32)
        return Operand(values=bf16_bits_to_f32(bits), stored=bits, dtype=dtype)
    if dtype == "f16":
        h = x32.astype(np.float16)  # numpy rounds to nearest even
        return Operand(values=h.astype(np.float32), stored=h, dtype=dtype)
    if dtype in FP8_DTYPES:
        # OCP fp8 (e4m3 without infinities, e5m2), rounded to nearest even by
        # torch's conversion; stored as the raw codes (uint8)
        import torch
        tdt = torch.float8_e4m3fn if dtype == "e4m3" else torch.float8_e5m2
        q = torch.from_numpy(x32).to(tdt)
        return Operand(values=q.to(torch.float32).numpy(),
                       stored=q.view(torch.uint8).numpy().copy(), dtype=dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw(rng: np.random.Generator, shape, dist: Tuple[str, float]) -> np.ndarray:
    kind, scale = dist
    if kind == "normal":  # scale is the standard deviation
        return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)
    if kind == "uniform":  # U(-scale, scale)
        u = rng.random(size=shape, dtype=np.float32)
        return (u * np.float32(2.0) - np.float32(1.0)) * np.float32(scale)
    raise ValueError(f"unknown distribution {kind!r}")


def filter_std(s: Shape) -> float:
    return float(1.0 / np.sqrt(s.fh * s.fw))


@dataclasses.dataclass
class Inputs:
    shape: Shape
    dtype: str
    x: Operand
    w: Operand
    dy: Optional[Operand]


def make_inputs(
    s: Shape,
    dtype: str = "f32",
    seed: int = 0,
    x_dist: Tuple[str, float] = ("normal", 1.0),
    w_dist: Optional[Tuple[str, float]] = None,
    dy_dist: Optional[Tuple[str, float]] = ("normal", 1.0),
) -> Inputs:
    """Draw X, W, dY (in that order) for shape ``s``."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    if w_dist is None:
        w_dist = ("normal", filter_std(s))
    rng = np.random.default_rng(seed)
    x = to_operand(_draw(rng, s.x_shape(), x_dist), dtype)
    w = to_operand(_draw(rng, s.w_shape(), w_dist), dtype)
    dy = None
    if dy_dist is not None:
        dy = to_operand(_draw(rng, s.y_shape(), dy_dist), dtype)
    return Inputs(shape=s, dtype=dtype, x=x, w=w, dy=dy)


# --------------------------------------------------------------------------
# Named workloads.  Each entry: shapes, operand distributions, ops, dtypes.
# --------------------------------------------------------------------------

def _same(n, hw, c, f, stride=1):
    p = (f - 1) // 2
    return Shape(n, hw, hw, c, f, f, stride, stride, p, p)


SWEEP_FILTERS = (3, 5, 7, 9, 13, 17, 21, 27, 31)
SWEEP_STAGES = ((56, 128), (28, 256), (14, 512), (7, 1024))

WORKLOADS: Dict[str, dict] = {
    # Small forward check: N=1, 14x14, C=32, 7x7, stride 1, pad 3, U(-1,1).
    "fwd_n1_14x14_c32_k7": dict(
        shapes=[_same(1, 14, 32, 7)],
        x_dist=("uniform", 1.0), w_dist=("uniform", 1.0),
        ops=("fwd",), dtypes=("f32",)),
    # CNN-stage forward: N=64, 56x56, C=128, 7x7, pad 3, stride 1 and 2.
    "fwd_n64_56x56_c128_k7": dict(
        shapes=[_same(64, 56, 128, 7), _same(64, 56, 128, 7, stride=2)],
        x_dist=("normal", 1.0), w_dist=None,
        ops=("fwd",), dtypes=("f32",)),
    # Large filter, all three ops: N=32, 56x56, C=128, 31x31, pad 15.
    "all_n32_56x56_c128_k31": dict(
        shapes=[_same(32, 56, 128, 31)],
        x_dist=("normal", 1.0), w_dist=None,
        ops=("fwd", "bwd_data", "bwd_filter"), dtypes=("f32",)),
    # Filter-size sweep at four stage shapes, N=64, all three ops.
    "sweep_n64_stages": dict(
        shapes=[_same(64, hw, c, f) for (hw, c) in SWEEP_STAGES for f in SWEEP_FILTERS],
        x_dist=("normal", 1.0), w_dist=None,
        ops=("fwd", "bwd_data", "bwd_filter"), dtypes=("f32",)),
    # Strided backward of the CNN stage's stride-2 forward (N=64, 56x56,
    # C=128, 7x7, pad 3): the data and filter gradients a training step needs.
    "strided_bwd_n64_56x56_c128_k7_s2": dict(
        shapes=[_same(64, 56, 128, 7, stride=2)],
        x_dist=("normal", 1.0), w_dist=None,
        ops=("bwd_data", "bwd_filter"), dtypes=("f32",)),
    # Mixed precision: bf16/fp16 operands, fp32 accumulate/output.
    "mixed_n128_28x28_c512": dict(
        shapes=[_same(128, 28, 512, 13), _same(128, 28, 512, 31)],
        x_dist=("normal", 1.0), w_dist=None,
        ops=("fwd", "bwd_data", "bwd_filter"), dtypes=("bf16", "f16")),
    # Low-bit operands on the same shapes: OCP fp8 (e4m3, e5m2) operands,
    # fp32 accumulate/output.
    "lowbit_n128_28x28_c512": dict(
        shapes=[_same(128, 28, 512, 13), _same(128, 28, 512, 31)],
        x_dist=("normal", 1.0), w_dist=None,
        ops=("fwd", "bwd_data", "bwd_filter"), dtypes=("e4m3", "e5m2")),
}

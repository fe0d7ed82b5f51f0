"""Host-side checks of the benchmark's model: buffer rotation and the
algorithmic byte and flop counts it divides by (no GPU)."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dwc_inputs import WORKLOADS, Shape  # noqa: E402


def _plans():
    yield "headline", bench.headline_plan(), "f32"
    for name, wl in WORKLOADS.items():
        for s in wl["shapes"]:
            for dt in wl["dtypes"]:
                yield name, [(s, op) for op in wl["ops"]], dt


@pytest.mark.parametrize("name,plan,dtype", list(_plans()),
                         ids=lambda v: v if isinstance(v, str) else "")
def test_every_op_rotates_over_a_gibibyte(name, plan, dtype):
    """Each op of a plan, launched alone on consecutive buffer sets, cycles
    through at least ROTATE_BYTES before it reuses a set (so no timed
    launch reads operands a previous launch left in the 256 MB Infinity
    Cache), unless the 16-set cap is reached."""
    n = bench.rotation_sets(plan, dtype)
    for s, op in plan:
        b = bench.op_model(s, op, dtype)["bytes"]
        assert n == 16 or n * b >= bench.ROTATE_BYTES, (name, op, n, b)


def test_headline_op_model():
    """Flops and bytes of the CNN-stage step, counted by hand: 2*N*OH*OW*C*49
    flops per op; fp32 X (or dY) in and the output out."""
    plan = bench.headline_plan()
    n, h, c = 64, 56, 128
    px = n * h * h * c
    flops_s1 = 2 * px * 49
    m = {(s.stride_h, op): bench.op_model(s, op, "f32") for s, op in plan}
    assert m[(1, "fwd")]["flops"] == flops_s1
    assert m[(2, "fwd")]["flops"] == flops_s1 // 4
    assert m[(1, "bwd_data")]["flops"] == flops_s1
    assert m[(1, "bwd_filter")]["flops"] == flops_s1
    assert m[(1, "fwd")]["bytes"] == 4 * (px + 49 * c) + 4 * px
    assert m[(2, "fwd")]["bytes"] == 4 * (px + 49 * c) + 4 * px // 4
    assert m[(1, "bwd_filter")]["bytes"] == 4 * 2 * px + 4 * 49 * c

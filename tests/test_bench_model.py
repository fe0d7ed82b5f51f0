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
    yield "headline", bench.headline_plan(), bench.HEADLINE_DTYPE
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
    Cache), unless the 64-set cap is reached."""
    n = bench.rotation_sets(plan, dtype)
    for s, op in plan:
        b = bench.op_model(s, op, dtype)["bytes"]
        assert n == 64 or n * b >= bench.ROTATE_BYTES, (name, op, n, b)


def test_headline_op_model():
    """Flops and bytes of the mixed-precision step (N=128, 28x28, C=512,
    31x31, pad 15, fp16 operands), counted by hand: 2*N*OH*OW*C*961 flops
    per op; 2-byte operands in, the fp32 output out."""
    plan = bench.headline_plan()
    assert [op for _, op in plan] == ["fwd", "bwd_data", "bwd_filter"]
    assert bench.HEADLINE_DTYPE == "f16"
    n, h, c, f = 128, 28, 512, 31
    px = n * h * h * c
    flops = 2 * px * f * f
    m = {op: bench.op_model(s, op, "f16") for s, op in plan}
    for op in m:
        assert m[op]["flops"] == flops
        assert m[op]["bound"] == "mfma" and m[op]["roofline"] == bench.PEAK_BF16_MFMA
    assert m["fwd"]["bytes"] == 2 * (px + f * f * c) + 4 * px
    assert m["bwd_data"]["bytes"] == 2 * (px + f * f * c) + 4 * px
    assert m["bwd_filter"]["bytes"] == 2 * 2 * px + 4 * f * f * c
    # eta_D of the forward: flops over operand elements (~1904 for 31x31)
    assert abs(m["fwd"]["eta_d"] - flops / (px + f * f * c)) < 1e-9


def test_config_entries_cover_every_configuration():
    """The per-configuration entries: all five configurations (c4's 36
    points with all three ops, c5's two filters in bf16 and fp16 on both
    kernel families) and the strided-backward and fp8 rows."""
    cases = list(bench.config_cases())
    tags = {bench.config_label(n, s, dt)[0] for n, s, dt, _, _ in cases}
    assert tags == {"c1", "c2", "c3", "c4", "c5", "f1", "f4"}
    c4 = [c for c in cases if c[0] == "sweep_n64_stages"]
    assert len(c4) == 36 * 3
    c5 = [c for c in cases if c[0] == "mixed_n128_28x28_c512"]
    assert len(c5) == 2 * 2 * 3 * 2
    # compact form: c4 as per-stage lists over the nine filters
    recs = [{"config": bench.config_label(n, s, dt)[0], "case": bench.config_label(n, s, dt)[1],
             "op": op, "algo": algo, "ms": 0.1, "roofline_frac": 0.5}
            for n, s, dt, op, algo in cases]
    out = bench.compact_configs(recs)
    assert out["c4"]["filters"] == list(bench.SWEEP_FILTERS)
    assert len(out["c4"]["56x56c128"]["bwd_filter.frac"]) == 9
    assert len(out["c4"]["7x7c1024"]["fwd.us"]) == 9
    assert set(out["c5"]["28x28c512k31s1-f16"]) == {"fwd", "bwd_data", "bwd_filter",
                                                     "fwd@vector", "bwd_data@vector",
                                                     "bwd_filter@vector"}
    import json
    assert len(json.dumps(out, separators=(",", ":"))) < 4000

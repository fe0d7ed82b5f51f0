"""The C ABI without a GPU: the library loads, exports every function that
include/dwc.h declares, and rejects bad calls before touching the device."""

import ctypes
import json
import os
import re

import pytest

import depthwise_convolution_dwc_amd as dwc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dwc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dwc.LIB_PATH),
                                reason="libdwc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dwc_[a-z_]+)\s*\(", text)))


def test_header_declares_the_python_list():
    assert declared_functions() == sorted(dwc.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dwc.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_the_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {dwc.LIB_PATH}").read().split("\n")
    names = {ln.split()[-1] for ln in out if " T " in ln}
    assert names == set(declared_functions())


def test_version_and_strings():
    assert dwc.lib().dwc_version() == 100
    assert dwc.lib().dwc_status_string(0) == b"ok"
    assert dwc.lib().dwc_status_string(5) == b"output aliases an input"


def test_struct_layout_matches_header():
    # int64 x4 + int32 x10 = 72 bytes, no padding
    assert ctypes.sizeof(dwc.Problem) == 72


@pytest.mark.parametrize("n,h,f,s,p,want", [
    (1, 14, 7, 1, 3, (14, 14)), (64, 56, 7, 2, 3, (28, 28)), (32, 56, 31, 1, 15, (56, 56)),
    (64, 7, 31, 1, 15, (7, 7)), (1, 3, 3, 2, 1, (2, 2)), (2, 5, 5, 1, 0, (1, 1))])
def test_output_dims(n, h, f, s, p, want):
    assert dwc.output_dims(dwc.problem(n, h, h, 8, f, f, s, p)) == want


BAD = [
    (dict(n=-1), 1), (dict(h=0), 1), (dict(c=0), 1), (dict(fh=0), 1),
    (dict(stride=0), 1), (dict(pad=-1), 1), (dict(dtype=7), 1), (dict(dtype=5), 1),
    (dict(h=3, fh=7, pad=1), 1),  # filter larger than padded input
    (dict(algo=9), 1), (dict(wgrad_split=-2), 1),
]


@pytest.mark.parametrize("change,status", BAD)
def test_bad_parameters_rejected(change, status):
    kw = dict(n=2, h=9, w=9, c=16, fh=3, fw=3, stride=1, pad=1, dtype=0, algo="auto",
              wgrad_split=0)
    kw.update(change)
    if "stride" in change:
        kw["stride"] = change["stride"]
    p = dwc.problem(kw["n"], kw["h"], kw["w"], kw["c"], kw["fh"], kw.get("fw", kw["fh"]),
                    kw["stride"], kw["pad"], kw["dtype"], kw["algo"], kw["wgrad_split"])
    for op in (0, 1, 2):
        assert dwc.check(p, op) == status
    assert dwc.last_error() != ""


def test_fp32_output_required():
    p = dwc.problem(1, 8, 8, 4, 3, 3, 1, 1)
    p.out_dtype = 1
    assert dwc.check(p, 0) == 2


def test_direct_unavailable_is_unsupported():
    # width 33 is past every register-window kernel; forcing it is an error,
    # auto falls back
    p = dwc.problem(1, 40, 40, 4, 33, 33, 1, 1, algo="direct")
    assert dwc.check(p, 0) == 2
    p = dwc.problem(1, 40, 40, 4, 33, 33, 1, 1, algo="auto")
    assert dwc.check(p, 0) == 0
    assert "generic" in dwc.plan_describe(p, 0)
    # stride-2 data gradient runs the phase kernel, or the gather kernel
    # when asked for the generic family
    p = dwc.problem(1, 8, 8, 4, 3, 3, 2, 1)
    assert "bwd_data phase" in dwc.plan_describe(p, 1)
    p = dwc.problem(1, 8, 8, 4, 3, 3, 2, 1, algo="generic")
    assert "bwd_data generic" in dwc.plan_describe(p, 1)


def test_plans_for_the_named_workloads():
    p = dwc.problem(64, 56, 56, 128, 7, 7, 1, 3)
    d = dwc.plan_describe(p, 0)
    assert d.startswith("fwd sweep") and "strip=7" in d
    assert dwc.plan_describe(p, 1).startswith("bwd_data sweep")
    d = dwc.plan_describe(p, 2)
    assert d.startswith("bwd_filter sweep")
    p = dwc.problem(32, 56, 56, 128, 31, 31, 1, 15)
    d = dwc.plan_describe(p, 0)
    assert d.startswith("fwd mfma dt=f32") and " f32=1 fwi=31 t=7 img=0 " in d, d
    assert " rg=14 cg=2 tiles=896 " in d and " same=1 " in d, d
    assert dwc.plan_describe(p, 1).startswith("bwd_data mfma dt=f32")
    d = dwc.plan_describe(p, 2)
    assert d.startswith("bwd_filter mfma dt=f32") and " tw=8 nb=14 cg=1 nw=8 " in d, d
    p = dwc.problem(64, 56, 56, 128, 7, 7, 2, 3)
    assert "sw=2" in dwc.plan_describe(p, 0)
    p = dwc.problem(128, 28, 28, 512, 13, 13, 1, 6, dtype=dwc.BF16)
    assert "dt=bf16" in dwc.plan_describe(p, 0)


def test_fp32_mfma_plans_and_rejections(monkeypatch):
    monkeypatch.delenv("DWC_MFMA_F32", raising=False)
    # AUTO: large filters on outputs at least 24 wide; on outputs at most 16
    # wide, 21x21 and up (width 7: 27x27 and up) where the images kernel has
    # 8 waves per CU, and wherever the vector kernel has fewer; the vector
    # kernels elsewhere
    for (n, h, c, f, want, img) in ((64, 56, 128, 13, True, 0), (64, 28, 256, 31, True, 0),
                                    (64, 14, 512, 31, True, 1), (64, 14, 512, 21, True, 1),
                                    (64, 14, 512, 17, False, 0), (64, 7, 1024, 31, True, 1),
                                    (64, 7, 1024, 21, False, 0), (64, 56, 128, 9, False, 0),
                                    (32, 14, 512, 31, True, 0), (32, 14, 512, 13, True, 0),
                                    (8, 14, 512, 31, True, 0), (64, 14, 1024, 13, False, 0),
                                    (16, 14, 256, 21, True, 0), (64, 20, 256, 21, False, 0)):
        p = dwc.problem(n, h, h, c, f, f, 1, f // 2)
        d = dwc.plan_describe(p, 0)
        assert (" f32=1 " in d) == want, (n, h, c, f, d)
        if want:
            assert f" img={img} " in d, (n, h, c, f, d)
    # the images kernel: 4 tiles per wave above width 8, else 2
    d = dwc.plan_describe(dwc.problem(64, 14, 14, 512, 31, 31, 1, 15), 0)
    assert " t=4 img=1 rg=4 cg=1 tiles=64 " in d, d  # 16 image groups x 4 row groups
    d = dwc.plan_describe(dwc.problem(64, 7, 7, 1024, 27, 27, 1, 13), 0)
    assert " t=2 img=1 rg=2 cg=1 tiles=32 " in d, d
    # fewer than 4 images, or too few waves: the rows kernel
    d = dwc.plan_describe(dwc.problem(3, 14, 14, 512, 31, 31, 1, 15), 0)
    assert " img=0 " in d, d
    monkeypatch.setenv("DWC_MFMA_F32_IMG", "1")
    d = dwc.plan_describe(dwc.problem(6, 14, 14, 16, 21, 21, 1, 10, algo="mfma"), 0)
    assert " t=4 img=1 rg=4 cg=1 tiles=8 " in d, d
    d = dwc.plan_describe(dwc.problem(3, 14, 14, 16, 21, 21, 1, 10, algo="mfma"), 0)
    assert " img=0 " in d, d
    monkeypatch.setenv("DWC_MFMA_F32_IMG", "0")
    assert " img=0 " in dwc.plan_describe(dwc.problem(64, 14, 14, 512, 31, 31, 1, 15), 0)
    monkeypatch.delenv("DWC_MFMA_F32_IMG")
    # the band width rounds the filter width up; tiles per wave and groups
    d = dwc.plan_describe(dwc.problem(2, 12, 20, 16, 5, 11, 1, (2, 3), algo="mfma"), 0)
    assert " fw=11 fh=5 " in d and " fwi=13 " in d and " same=0 " in d, d
    # width 57: four right-aligned 16-column groups issue fewer instructions
    # than three 28-column ones (the last two overlapping in 27 columns)
    d = dwc.plan_describe(dwc.problem(2, 30, 57, 16, 21, 21, 1, 10, algo="mfma"), 0)
    assert " t=4 img=0 " in d and " cg=4 " in d and " rg=8 " in d and " same=1 " in d, d
    monkeypatch.setenv("DWC_MFMA_F32_T", "2")
    d = dwc.plan_describe(dwc.problem(2, 30, 57, 16, 21, 21, 1, 10, algo="mfma"), 0)
    assert " t=2 " in d and " cg=8 " in d, d
    monkeypatch.delenv("DWC_MFMA_F32_T")
    # the band of 64 filter rows of width 31 fits one CU's LDS
    d = dwc.plan_describe(dwc.problem(1, 70, 40, 16, 64, 31, 1, 0, algo="mfma"), 0)
    assert " lds=151552 " in d, d
    # rejections: C % 16, FW > 31, FH > 64, stride 2, half precision
    for args, kw in (((1, 20, 20, 24, 13, 13, 1, 6), {}), ((1, 40, 40, 16, 32, 32, 1, 0), {}),
                     ((1, 70, 8, 16, 65, 3, 1, 0), {}), ((1, 20, 20, 16, 13, 13, 2, 6), {})):
        p = dwc.problem(*args, algo="mfma")
        assert dwc.check(p, 0) == 2, args  # DWC_ERR_UNSUPPORTED
    monkeypatch.setenv("DWC_MFMA_F32", "0")
    assert " f32=1 " not in dwc.plan_describe(dwc.problem(32, 56, 56, 128, 31, 31, 1, 15), 0)


def test_fp32_mfma_wgrad_plans(monkeypatch):
    monkeypatch.delenv("DWC_MFMA_F32", raising=False)
    # AUTO: 4x4 tiles at least 85% real taps (64% up to 16 columns), 12+
    # rows and columns, outputs wider than 8 unless the filter is 29+ or at
    # most 16 wide
    for (h, c, f, want) in ((56, 128, 31, True), (28, 256, 27, True), (56, 128, 17, False),
                            (56, 128, 21, False), (7, 1024, 27, False), (7, 1024, 31, True),
                            (56, 128, 16, True), (56, 128, 9, False), (56, 128, 13, True),
                            (7, 1024, 13, True)):
        p = dwc.problem(64, h, h, c, f, f, 1, f // 2)
        d = dwc.plan_describe(p, 2)
        assert (" f32=1 " in d) == want, (h, f, d)
    # one column group per 56 output columns; the requested split is the
    # number of row slices; slices times column groups partials
    d = dwc.plan_describe(dwc.problem(2, 10, 70, 16, 21, 21, 1, 10, algo="mfma", wgrad_split=7), 2)
    assert " tw=6 nb=14 cg=2 nw=6 rps=3 zr=7 z=14 " in d, d
    p = dwc.problem(2, 10, 70, 16, 21, 21, 1, 10, algo="mfma", wgrad_split=7)
    assert dwc.workspace_size(p) == (7 * 2 * 21 * 21 * 16 * 4 + 255) // 256 * 256
    d = dwc.plan_describe(dwc.problem(5, 6, 40, 16, 1, 31, 1, (0, 15), algo="mfma"), 2)
    assert " tw=8 nb=14 " in d and " nw=3 " in d, d  # three waves to stage a row
    # rejections: C % 16, FH or FW > 32, stride 2
    for args in ((1, 20, 20, 24, 13, 13, 1, 6), (1, 40, 40, 16, 33, 3, 1, 0),
                 (1, 40, 40, 16, 3, 33, 1, 0), (1, 20, 20, 16, 13, 13, 2, 6)):
        assert dwc.check(dwc.problem(*args, algo="mfma"), 2) == 2, args


def test_workspace_size_matches_split():
    # the vector kernels: one partial per slice, none for one slice
    p = dwc.problem(32, 56, 56, 128, 31, 31, 1, 15, wgrad_split=8, algo="direct")
    assert dwc.workspace_size(p) == 8 * 31 * 31 * 128 * 4
    p = dwc.problem(32, 56, 56, 128, 31, 31, 1, 15, wgrad_split=1, algo="direct")
    assert dwc.workspace_size(p) == 0
    # the matrix-core kernels always write partials (one per slice)
    p = dwc.problem(32, 56, 56, 128, 31, 31, 1, 15, wgrad_split=8)
    assert dwc.workspace_size(p) == 8 * 31 * 31 * 128 * 4
    p = dwc.problem(32, 56, 56, 128, 31, 31, 1, 15, wgrad_split=1)
    assert dwc.workspace_size(p) == (31 * 31 * 128 * 4 + 255) // 256 * 256
    p = dwc.problem(0, 56, 56, 128, 31, 31, 1, 15)
    assert dwc.workspace_size(p) == 0
    p = dwc.problem(2, 8, 8, 4, 3, 3, 1, 1, wgrad_split=17)  # > N*OH = 16
    assert dwc.check(p, 2) == 1


def test_pointer_errors_are_reported_before_any_launch():
    # Fake addresses: every call below must fail validation, so nothing is
    # launched and no GPU is needed.
    p = dwc.problem(1, 8, 8, 16, 3, 3, 1, 1)
    L = dwc.lib()
    pp = ctypes.byref(p)
    assert L.dwc_fwd(pp, 0x10000, 0x20000, None, None) == 1           # null output
    assert L.dwc_fwd(pp, None, 0x20000, 0x30000, None) == 1           # null input
    assert L.dwc_fwd(pp, 0x10001, 0x20000, 0x30000, None) == 3        # misaligned x
    assert L.dwc_fwd(pp, 0x10000, 0x20000, 0x30002, None) == 3        # misaligned y
    x = 0x100000
    assert L.dwc_fwd(pp, x, 0x200000, x + 64, None) == 5              # y overlaps x
    assert L.dwc_bwd_data(pp, x, 0x200000, x - 64, None) == 5         # dx overlaps dy
    q = dwc.problem(4, 32, 32, 64, 5, 5, 1, 2, wgrad_split=4)
    need = dwc.workspace_size(q)
    assert need > 0
    assert L.dwc_bwd_filter(ctypes.byref(q), 0x1000000, 0x3000000, 0x5000000, None, 0, None) == 4
    assert L.dwc_bwd_filter(ctypes.byref(q), 0x1000000, 0x3000000, 0x5000000, 0x6000000,
                            need - 4, None) == 4
    # workspace overlapping dW
    assert L.dwc_bwd_filter(ctypes.byref(q), 0x1000000, 0x3000000, 0x5000000, 0x5000000,
                            need, None) == 5
    half = dwc.problem(1, 8, 8, 16, 3, 3, 1, 1, dtype=dwc.BF16)
    assert L.dwc_fwd(ctypes.byref(half), 0x10001, 0x20000, 0x30000, None) == 3


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dwc, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(dwc, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        dwc.lib()


def test_mfma_plans_and_rejections(monkeypatch):
    p = dwc.problem(128, 28, 28, 512, 13, 13, 1, 6, dtype=dwc.BF16)
    assert dwc.plan_describe(p, 0).startswith("fwd mfma")
    assert dwc.plan_describe(p, 1).startswith("bwd_data mfma")
    assert dwc.plan_describe(p, 2).startswith("bwd_filter mfma")
    # 13x13: the row-packed kernel; 31x31: the batch-packed kernel (AUTO
    # takes it from 17 filter rows on, with widths up to 32): 16 images x 16
    # channels per workgroup (two 16-column output groups, four output
    # rows staged per round), or 32 x 8 when asked for
    assert " batch=1 " not in dwc.plan_describe(p, 0)
    p = dwc.problem(128, 28, 28, 512, 31, 31, 1, 15, dtype=dwc.F16)
    d = dwc.plan_describe(p, 0)
    assert d.startswith("fwd mfma") and " batch=1 cb=16 imgs=16 rows=7 ng=8 " in d, d
    assert " ocg=2 orows=4" in d and " blocks=1024" in d, d
    assert " batch=1 " in dwc.plan_describe(p, 1)
    monkeypatch.setenv("DWC_MFMA_BATCH_IMG", "32")
    d = dwc.plan_describe(p, 0)
    assert " batch=1 cb=8 imgs=32 rows=7 ng=4 " in d and " blocks=1024" in d, d
    monkeypatch.delenv("DWC_MFMA_BATCH_IMG")
    # the 16-image kernel from 8 images (one output group up to 16 columns)
    q = dwc.problem(8, 16, 16, 32, 17, 9, 1, (8, 4), dtype=dwc.BF16)
    assert " imgs=16 " in dwc.plan_describe(q, 0) and " ocg=1 " in dwc.plan_describe(q, 0)
    # C % 16 != 0: the 32-image kernel
    q = dwc.problem(32, 16, 16, 24, 17, 9, 1, (8, 4), dtype=dwc.BF16)
    assert " imgs=32 " in dwc.plan_describe(q, 0)
    for kw in (dict(n=4), dict(w=40)):
        a = dict(n=128, w=28, pad=15, **{})
        a.update(kw)
        q = dwc.problem(a["n"], 28, a["w"], 512, 31, 31, 1, a["pad"], dtype=dwc.F16)
        d = dwc.plan_describe(q, 0)
        assert d.startswith("fwd mfma") and " batch=1 " not in d, (kw, d)
    q = dwc.problem(128, 28, 28, 512, 31, 31, 1, 15, dtype=dwc.F16)
    q2 = dwc.problem(128, 28, 28, 512, 31, 15, 1, (15, 7), dtype=dwc.F16)
    assert " batch=1 " in dwc.plan_describe(q2, 0)  # FH decides, not FW
    del q
    d = dwc.plan_describe(p, 2)
    assert d.startswith("bwd_filter mfma") and "nfm=2" in d and "nfn=2" in d
    # the vector kernels stay reachable
    p = dwc.problem(128, 28, 28, 512, 13, 13, 1, 6, dtype=dwc.BF16, algo="direct")
    assert dwc.plan_describe(p, 0).startswith("fwd direct")
    assert dwc.plan_describe(p, 2).startswith("bwd_filter direct")
    # conditions of the packed kernels: half-precision operands (fp32: the
    # forward and data gradient, C a multiple of 16), stride 1, C a multiple
    # of 8, FW <= 32, output width <= 64 (forward), FH <= 32 (filter
    # gradient); 16-bit problems past them (outputs or inputs wider than 64)
    # with C a multiple of 16 run the fp32 matrix-core kernels, operands
    # widened as they are loaded
    base = dict(n=2, h=20, w=20, c=16, fh=5, fw=5, stride=1, pad=2, dtype=dwc.BF16)
    for kw, ops in ((dict(dtype=dwc.F32, c=24), (0, 1, 2)),
                    (dict(stride=2), (0, 1, 2)),
                    (dict(c=12), (0, 1, 2)), (dict(fw=33, pad=16), (0, 1, 2)),
                    (dict(w=80, c=8), (0, 2)), (dict(fh=33, pad=16), (2,))):
        a = dict(base, **kw)
        q = dwc.problem(a["n"], a["h"], a["w"], a["c"], a["fh"], a["fw"], a["stride"],
                        a["pad"], dtype=a["dtype"], algo="mfma")
        for op in ops:
            assert dwc.check(q, op) == 2, (kw, op)
            assert "packed-MFMA" in dwc.last_error()
    q = dwc.problem(2, 20, 20, 16, 5, 5, 1, 2, dtype=dwc.BF16, algo="mfma")
    assert dwc.check(q, 0) == 0 and dwc.check(q, 1) == 0 and dwc.check(q, 2) == 0
    for dt, name in ((dwc.BF16, "bf16"), (dwc.F16, "f16")):
        q = dwc.problem(2, 20, 80, 16, 5, 5, 1, 2, dtype=dt, algo="mfma")
        for op, opn in ((0, "fwd"), (1, "bwd_data"), (2, "bwd_filter")):
            d = dwc.plan_describe(q, op)
            assert d.startswith(f"{opn} mfma dt={name}") and " f32=1 " in d, d
    # AUTO: the bf16 filter gradient of 56-wide images with 13x13 filters
    # (past the packed kernel's LDS budget) takes it too; the 16-bit forward
    # only on request
    q = dwc.problem(64, 56, 56, 128, 13, 13, 1, 6, dtype=dwc.BF16)
    assert " f32=1 " in dwc.plan_describe(q, 2)
    q = dwc.problem(32, 112, 112, 64, 13, 13, 1, 6, dtype=dwc.BF16)
    assert dwc.plan_describe(q, 0).startswith("fwd direct")
    assert " f32=1 " in dwc.plan_describe(q, 2)
    # an empty batch plans (it only zero-fills dW) and needs no workspace
    q = dwc.problem(0, 20, 20, 16, 5, 5, 1, 2, dtype=dwc.BF16, algo="mfma")
    assert dwc.check(q, 2) == 0 and dwc.workspace_size(q) == 0


def test_mfma_wgrad_plan_geometry():
    """The packed filter gradient splits the batch into slices of whole images
    (one workspace partial per slice and channel block), never more slices than
    images, and AUTO's workspace also covers the vector fallback."""
    import re
    for n, split in ((128, 0), (3, 0), (5, 2), (7, 7), (7, 3)):
        p = dwc.problem(n, 28, 28, 512, 13, 13, 1, 6, dtype=dwc.BF16, algo="mfma",
                        wgrad_split=split)
        d = dict((k, int(v)) for k, v in re.findall(r"(\w+)=(\d+)", dwc.plan_describe(p, 2)))
        z, ipb = d["z"], d["ipb"]
        assert 1 <= z <= n and (z - 1) * ipb < n <= z * ipb
        if split:
            assert z <= split
        assert d["blocks"] == z * d["cblk"] == z * 512 // 8
        need = z * 13 * 13 * 512 * 4
        assert dwc.workspace_size(p) >= need
        pa = dwc.problem(n, 28, 28, 512, 13, 13, 1, 6, dtype=dwc.BF16, wgrad_split=split)
        pd = dwc.problem(n, 28, 28, 512, 13, 13, 1, 6, dtype=dwc.BF16, algo="direct",
                         wgrad_split=split)
        assert dwc.workspace_size(pa) >= max(need, dwc.workspace_size(pd))


def test_mfma_forced_misaligned_is_rejected_before_launch():
    p = dwc.problem(1, 8, 8, 16, 3, 3, 1, 1, dtype=dwc.BF16, algo="mfma")
    L = dwc.lib()
    assert L.dwc_fwd(ctypes.byref(p), 0x10002, 0x20000, 0x30000, None) == 3
    assert L.dwc_bwd_data(ctypes.byref(p), 0x10000, 0x20000, 0x30008, None) == 3
    ws = dwc.workspace_size(p)
    # the filter gradient also stores 16-byte partials into the workspace
    assert L.dwc_bwd_filter(ctypes.byref(p), 0x10000, 0x20000, 0x30000, 0x40008, ws + 64,
                            None) == 3


def test_strided_data_gradient_plans():
    """Equal strides >= 2 take the phase kernel (AUTO and DIRECT) while the
    sub-filter fits 16 x 16 taps; unequal strides and larger sub-filters
    take the generic kernel, and DIRECT is then an error."""
    p = dwc.problem(64, 56, 56, 128, 7, 7, 2, 3)
    d = dwc.plan_describe(p, 1)
    assert d.startswith("bwd_data phase") and "km=4" in d and "s=2" in d
    q = dwc.problem(1, 10, 10, 64, 5, 5, 3, 2, algo="direct")
    assert dwc.check(q, 1) == 0 and "km=2" in dwc.plan_describe(q, 1)
    big = dwc.problem(1, 40, 40, 8, 35, 35, 2, 17)
    assert dwc.plan_describe(big, 1).startswith("bwd_data generic")
    big.algo = dwc.ALGO["direct"]
    assert dwc.check(big, 1) == 2
    uneq = dwc.problem(1, 12, 12, 8, 3, 3, (2, 1), 1)
    assert dwc.plan_describe(uneq, 1).startswith("bwd_data generic")


def test_output_dims_do_not_depend_on_the_kernel_choice():
    """OH and OW come from the problem alone: a problem whose forced algo has
    no forward kernel (stride 3 forced to DIRECT) still has output dims, and
    its data gradient plans."""
    p = dwc.problem(1, 11, 13, 40, 3, 3, 3, 1, algo="direct")
    assert dwc.output_dims(p) == (4, 5)
    assert dwc.check(p, 0) == 2
    assert dwc.check(p, 1) == 0
    bad = dwc.problem(1, 4, 4, 8, 7, 7, 1, 0)
    with pytest.raises(dwc.DwcError):
        dwc.output_dims(bad)


def test_fwd_fused_rejections_before_any_launch():
    """The fused-prologue forward checks its activation, kernel family and
    scale/shift vectors synchronously; none of these calls launches."""
    L = dwc.lib()
    P = ctypes.byref
    X, W, Y, SC, SH = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    p = dwc.problem(2, 8, 8, 64, 3, 3, 1, 1)
    assert L.dwc_fwd_fused(P(p), X, SC, SH, 7, W, Y, None) == 1  # unknown activation
    assert "activation" in dwc.last_error()
    for algo in ("mfma", "generic"):
        q = dwc.problem(2, 8, 8, 64, 3, 3, 1, 1, algo=algo)
        assert L.dwc_fwd_fused(P(q), X, SC, SH, 1, W, Y, None) == 2
    for fh, fw, pad in ((11, 11, 5), (10, 10, 4), (3, 3, 1)):
        q = dwc.problem(2, 16, 16, 64, fh, fw, 3 if fw == 3 else 1, pad)
        assert L.dwc_fwd_fused(P(q), X, SC, SH, 1, W, Y, None) == 2, (fh, fw)
        assert "fused prologue" in dwc.last_error()
    assert L.dwc_fwd_fused(P(p), X, None, SH, 1, W, Y, None) == 1       # NULL scale
    assert L.dwc_fwd_fused(P(p), X, SC + 2, SH, 1, W, Y, None) == 3     # misaligned
    assert L.dwc_fwd_fused(P(p), X, Y + 64, SH, 1, W, Y, None) == 5     # scale inside y
    empty = dwc.problem(0, 8, 8, 64, 3, 3, 1, 1)
    assert L.dwc_fwd_fused(P(empty), None, None, None, 3, None, None, None) == 0
    # a 9-wide filter at stride 2, a tall 31 x 9 filter and even or 1-wide
    # filters (on the next wider body) are accepted
    for q in (dwc.problem(1, 16, 16, 64, 9, 9, 2, 4), dwc.problem(1, 40, 16, 64, 31, 9, 1, 4),
              dwc.problem(1, 16, 16, 64, 4, 4, 1, 1), dwc.problem(1, 16, 16, 64, 1, 1, 2, 0),
              dwc.problem(1, 16, 16, 64, 8, 8, 1, 3)):
        assert L.dwc_fwd_fused(P(q), X, SC + 2, SH, 0, W, Y, None) == 3  # reaches the checks


def test_hybrid_accumulation_plans():
    """DWC_ALGO_HYBRID: the filter gradient of fp16 operands on the sweep
    kernels only; everything else is DWC_ERR_UNSUPPORTED before a launch."""
    ok = dwc.problem(64, 56, 56, 128, 7, 7, 1, 3, dtype=dwc.F16, algo="hybrid")
    assert dwc.check(ok, 2) == 0
    d = dwc.plan_describe(ok, 2)
    assert d.startswith("bwd_filter sweep") and d.endswith("hybrid=1")
    assert dwc.workspace_size(ok) > 0
    assert "hybrid" not in dwc.plan_describe(dwc.problem(64, 56, 56, 128, 7, 7, 1, 3,
                                                         dtype=dwc.F16), 2)
    for kw, op in ((dict(dtype=dwc.F32), 2), (dict(dtype=dwc.BF16), 2), (dict(), 0), (dict(), 1),
                   (dict(fh=5, fw=3), 2), (dict(stride=2), 2), (dict(fh=11, fw=11, pad=5), 2)):
        a = dict(fh=7, fw=7, stride=1, pad=3, dtype=dwc.F16)
        a.update(kw)
        q = dwc.problem(8, 20, 20, 64, a["fh"], a["fw"], a["stride"], a["pad"], dtype=a["dtype"],
                        algo="hybrid")
        assert dwc.check(q, op) == 2, (kw, op)
        assert "hybrid accumulation" in dwc.last_error()


def test_fp8_operand_plans():
    """fp8 operands (one byte per element): the vector, sweep, phase and
    generic kernels take them for every shape; the planner reports the
    dtype; workspace sizes count one-byte operands like any other."""
    for dt, name in ((dwc.FP8_E4M3, "e4m3"), (dwc.FP8_E5M2, "e5m2")):
        for shape, op, kind in (((16, 80, 80, 128, 7, 7, 1, 3), 0, "sweep"),
                                ((64, 56, 56, 128, 7, 7, 2, 3), 0, "direct"),
                                ((64, 56, 56, 128, 7, 7, 2, 3), 1, "phase"),
                                ((16, 80, 80, 128, 7, 7, 1, 3), 2, "sweep"),
                                ((2, 9, 9, 8, 4, 6, 3, 1), 0, "generic")):
            p = dwc.problem(*shape, dtype=dt)
            assert dwc.check(p, op) == 0, (name, shape, op)
            d = dwc.plan_describe(p, op)
            assert name in d and kind in d, d
        for algo in ("direct", "generic"):
            p = dwc.problem(2, 9, 9, 16, 3, 3, 1, 1, dtype=dt, algo=algo)
            assert all(dwc.check(p, op) == 0 for op in (0, 1, 2))
        hy = dwc.problem(64, 56, 56, 128, 7, 7, 1, 3, dtype=dt, algo="hybrid")
        assert dwc.check(hy, 2) == 2


def test_fp8_mfma_plans_and_rejections():
    """The packed fp8 kernels, 16 channels per workgroup, C a multiple of
    16, stride 1, FW <= 32: the 16-image batch-packed kernel (16x16x32 fp8
    MFMAs) from 5 filter rows on, where widths are up to 32, within one
    CU's LDS; otherwise the row-packed kernel (16x16x128 MFMAs over four
    filter rows, output width <= 64, LDS within its per-workgroup limit)."""
    for dt, name in ((dwc.FP8_E4M3, "e4m3"), (dwc.FP8_E5M2, "e5m2")):
        for f in (3, 7, 13, 17, 31):
            p = dwc.problem(128, 28, 28, 512, f, f, 1, f // 2, dtype=dt, algo="mfma")
            for op in (0, 1):
                d = dwc.plan_describe(p, op)
                assert d.startswith(("fwd mfma", "bwd_data mfma")), d
                g = dict(kv.split("=") for kv in d.split()[2:])
                assert g["dt"] == name and g["cb"] == "16" and g["flip"] == str(op)
                if f >= 5:
                    assert g.get("batch") == "1" and g["imgs"] == "16", d
                    assert int(g["lds"]) <= 163840
                else:
                    assert "batch" not in g, d
                    assert int(g["lds"]) <= 81920
                    assert int(g["wp"]) % 16 == 0
                    assert int(g["wt"]) == 16 * (int(g["gt"]) + int(g["nf"]))
        for kw in (dict(c=24), dict(stride=2), dict(fw=33, fh=3, pad=(1, 16), w=40), dict(w=80, h=20)):
            a = dict(n=2, h=20, w=20, c=32, fh=5, fw=5, stride=1, pad=2)
            a.update(kw)
            q = dwc.problem(a["n"], a["h"], a["w"], a["c"], a["fh"], a["fw"], a["stride"],
                            a["pad"], dtype=dt, algo="mfma")
            assert dwc.check(q, 0) == 2, kw
            assert "no packed-MFMA kernel" in dwc.last_error()


def test_fp8_mfma_wgrad_plans():
    """The packed fp8 filter gradient: kWgmCb (8) channels per workgroup,
    dY rows padded so that every 36-byte band read stays in its row, X row
    pitch an odd number of 16-byte units, LDS within the limit."""
    for dt in (dwc.FP8_E4M3, dwc.FP8_E5M2):
        for f in (3, 7, 13, 31):
            p = dwc.problem(128, 28, 28, 512, f, f, 1, f // 2, dtype=dt, algo="mfma")
            d = dwc.plan_describe(p, 2)
            assert d.startswith("bwd_filter mfma"), d
            g = dict(kv.split("=") for kv in d.split()[2:])
            nk, nfm = int(g["nk"]), int(g["nfm"])
            assert int(g["cb"]) == 8 and (int(g["xp"]) // 16) % 2 == 1
            assert int(g["dyp"]) % 16 == 0
            assert int(g["dyp"]) >= 32 * nk + f // 2 + int(g["dpad"]) + 4
            assert int(g["dpad"]) + f // 2 >= 16 * (nfm - 1) + 15
            assert int(g["lds"]) <= 81920
        q = dwc.problem(2, 20, 80, 16, 5, 5, 1, 2, dtype=dt, algo="mfma")
        assert dwc.check(q, 2) == 2


def _header_enum(prefix):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"\b(" + prefix + r"[A-Z0-9_]+)\s*=\s*(\d+)", text)}


def test_algo_codes_match_the_header():
    """The binding's algo names map to the header's dwc_algo values: AUTO 0,
    VECTOR (= DIRECT) 1, MFMA 2, then GENERIC 3 and HYBRID 4."""
    h = _header_enum("DWC_ALGO_")
    assert h == {"DWC_ALGO_AUTO": 0, "DWC_ALGO_VECTOR": 1, "DWC_ALGO_DIRECT": 1,
                 "DWC_ALGO_MFMA": 2, "DWC_ALGO_GENERIC": 3, "DWC_ALGO_HYBRID": 4}
    for name, code in dwc.ALGO.items():
        assert h["DWC_ALGO_" + name.upper()] == code
    # algo 2 asks for the packed-MFMA kernels: bf16 at stride 1 has them,
    # fp32 for the forward-type ops only, and not at stride 2
    p = dwc.problem(1, 16, 16, 16, 5, 5, 1, 2, dtype=dwc.BF16, algo=2)
    assert dwc.check(p, 0) == 0 and " mfma " in dwc.plan_describe(p, 0)
    q = dwc.problem(1, 16, 16, 16, 5, 5, 1, 2, dtype=dwc.F32, algo=2)
    assert dwc.check(q, 0) == 0 and " f32=1 " in dwc.plan_describe(q, 0)
    assert dwc.check(q, 2) == 0 and " f32=1 " in dwc.plan_describe(q, 2)
    q = dwc.problem(1, 16, 16, 16, 5, 5, 2, 2, dtype=dwc.F32, algo=2)
    assert dwc.check(q, 0) == 2


def test_dtype_and_status_codes_match_the_header():
    d = _header_enum("DWC_")
    assert (d["DWC_F32"], d["DWC_BF16"], d["DWC_F16"], d["DWC_FP8_E4M3"], d["DWC_FP8_E5M2"]) == \
        (dwc.F32, dwc.BF16, dwc.F16, dwc.FP8_E4M3, dwc.FP8_E5M2)
    assert [d[k] for k in ("DWC_OK", "DWC_ERR_BAD_PARAM", "DWC_ERR_UNSUPPORTED",
                           "DWC_ERR_MISALIGNED", "DWC_ERR_WORKSPACE", "DWC_ERR_ALIAS",
                           "DWC_ERR_HIP")] == list(range(7))


def test_h4_plans(monkeypatch):
    """The 16-bit 4x4x4 kernel (fwd_mfma_h4n): AUTO on outputs up to 16
    wide with 9x9 to 13x13 filters while its waves fill the GPU; its tile
    shape; fp32 and fp8 never take it."""
    monkeypatch.delenv("DWC_MFMA_H4", raising=False)
    for (n, h, c, f, want) in ((64, 14, 512, 13, True), (64, 7, 1024, 9, True),
                               (64, 14, 512, 17, False), (64, 28, 256, 13, False),
                               (16, 14, 512, 13, False), (64, 14, 512, 7, False),
                               (128, 28, 512, 13, False)):
        for dt in (dwc.BF16, dwc.F16):
            d = dwc.plan_describe(dwc.problem(n, h, h, c, f, f, 1, f // 2, dtype=dt), 0)
            assert (" h4=1 " in d) == want, (n, h, c, f, d)
    d = dwc.plan_describe(dwc.problem(64, 14, 14, 512, 13, 13, 1, 6, dtype=dwc.BF16), 1)
    assert d.startswith("bwd_data mfma") and " flip=1 h4=1 fwi=13 t=4 " in d, d
    # 16 image groups x 4 row groups; the band (13 x 4 steps x 512 bytes) and
    # 8 row buffers of 4 images x 34 columns x 32 bytes
    assert " rg=4 cg=1 tiles=64 nw=8 same=1 cblk=32 lds=61440 " in d, d
    for dt in (dwc.F32, dwc.FP8_E4M3):
        d = dwc.plan_describe(dwc.problem(64, 14, 14, 512, 13, 13, 1, 6, dtype=dt), 0)
        assert " h4=1 " not in d, d
    monkeypatch.setenv("DWC_MFMA_H4", "0")
    assert " h4=1 " not in dwc.plan_describe(dwc.problem(64, 14, 14, 512, 13, 13, 1, 6,
                                                         dtype=dwc.BF16), 0)
    # forced: every 16-bit stride-1 problem with C % 16 == 0 and FW <= 17
    monkeypatch.setenv("DWC_MFMA_H4", "1")
    d = dwc.plan_describe(dwc.problem(2, 30, 57, 16, 17, 17, 1, 8, dtype=dwc.F16), 0)
    assert " h4=1 fwi=17 t=7 rg=8 cg=3 " in d, d
    d = dwc.plan_describe(dwc.problem(2, 30, 57, 24, 17, 17, 1, 8, dtype=dwc.F16), 0)
    assert " h4=1 " not in d, d  # C % 16 != 0


def test_packed_wgrad_slices():
    """Packed filter gradients: where the slice partials are cheap, about
    four rounds of workgroups (N=128 28x28 C=512: 43 slices of 3 images at
    13x13 in 16 bits, 32 of 4 in fp8, 16 of 8 at 31x31 in 16 bits); where
    they are dear (fp8 31x31) the rounds-times-images choice; a requested
    split as it is."""
    def zs(f, dt, split=0):
        d = dwc.plan_describe(dwc.problem(128, 28, 28, 512, f, f, 1, f // 2, dtype=dt,
                                          wgrad_split=split), 2)
        return [t for t in d.split() if t.startswith(("z=", "ipb="))]
    assert zs(13, dwc.BF16) == ["z=43", "ipb=3"]
    assert zs(13, dwc.F16) == ["z=43", "ipb=3"]
    assert zs(31, dwc.F16) == ["z=16", "ipb=8"]
    assert zs(13, dwc.FP8_E4M3) == ["z=32", "ipb=4"]
    assert zs(31, dwc.FP8_E4M3) == ["z=8", "ipb=16"]
    assert zs(13, dwc.BF16, split=12) == ["z=12", "ipb=11"]
    # the partials of all slices stay within a sixth of the operand bytes
    x_dy = 128 * 28 * 28 * 512 * 2 * 2
    for f in (13, 31):
        p = dwc.problem(128, 28, 28, 512, f, f, 1, f // 2, dtype=dwc.F16)
        z = int(zs(f, dwc.F16)[0][2:])
        assert z * f * f * 512 * 4 <= x_dy / 6


def test_sweep_chunks_small_launches():
    """Sweep launches under one wave per CU take one-row chunks; larger ones
    keep chunks of at least F rows."""
    d = dwc.plan_describe(dwc.problem(1, 14, 14, 32, 7, 7, 1, 3), 0)
    assert " sweep " in d and " rows=1 cpi=14 " in d, d
    d = dwc.plan_describe(dwc.problem(64, 7, 7, 1024, 7, 7, 1, 3), 0)
    assert " rows=7 cpi=1 " in d, d
    d = dwc.plan_describe(dwc.problem(64, 56, 56, 128, 7, 7, 1, 3), 0)
    rows = int([t for t in d.split() if t.startswith("rows=")][0][5:])
    assert rows >= 7, d


def test_small_filters_stay_on_sweeps():
    """AUTO keeps 16-bit and fp8 problems with square filters up to 7x7 at
    stride 1 on the sweep kernels (all three operations); from 9x9 on, and
    with algo=mfma, the packed matrix-core kernels."""
    for dt in (dwc.BF16, dwc.F16, dwc.FP8_E4M3, dwc.FP8_E5M2):
        for f in (3, 5, 7, 9):
            p = dwc.problem(128, 28, 28, 512, f, f, 1, f // 2, dtype=dt)
            for op in (0, 1, 2):
                d = dwc.plan_describe(p, op)
                assert (" sweep " in d) == (f <= 7), (dt, f, op, d)
            q = dwc.problem(128, 28, 28, 512, f, f, 1, f // 2, dtype=dt, algo="mfma")
            assert " mfma " in dwc.plan_describe(q, 0)
    # fp32 keeps its own rules (the sweeps up to 9x9)
    d = dwc.plan_describe(dwc.problem(64, 56, 56, 128, 9, 9, 1, 4), 0)
    assert " sweep " in d, d


def test_batch_kernel_one_round():
    """16-bit batch-packed forward below 17 filter rows only where its
    workgroups make one round of at least 3/4 of the CUs (256 here)."""
    for (n, c, f, want) in ((64, 256, 9, True), (32, 512, 13, True), (16, 1024, 13, True),
                            (64, 512, 13, False), (32, 256, 13, False), (128, 512, 13, False),
                            (128, 512, 31, True)):
        d = dwc.plan_describe(dwc.problem(n, 28, 28, c, f, f, 1, f // 2, dtype=dwc.BF16), 0)
        assert (" batch=1 " in d) == want, (n, c, f, d)
    # with algo=mfma the rule picks between the packed kernels from 5 rows on
    for (f, want) in ((5, True), (3, False)):
        d = dwc.plan_describe(dwc.problem(64, 28, 28, 256, f, f, 1, f // 2, dtype=dwc.BF16,
                                          algo="mfma"), 0)
        assert (" batch=1 " in d) == want, (f, d)


def test_padded_direct_widths():
    """Filter widths between the instantiated direct widths run on the next
    wider body (its extra taps skipped): forward, stride-1 data gradient and
    filter gradient take the direct plan with kfw the narrowest listed width
    >= FW, for fp32 operands at stride 1 and 2 (no matrix-core kernel: C is
    not a multiple of 16); widths past 31 stay on the generic kernels."""
    listed = (3, 5, 7, 9, 13, 17, 21, 27, 31)
    for fw in range(1, 32):
        kfw = min(k for k in listed if k >= fw)
        for s in (1, 2):
            p = dwc.problem(2, 40, 40, 24, 6, fw, s, (2, fw // 2), algo="direct")
            for op in ((0, 1, 2) if s == 1 else (0, 2)):
                d = dwc.plan_describe(p, op)
                g = dict(kv.split("=") for kv in d.split()[2:] if "=" in kv)
                assert d.split()[1] == "direct" and g["fw"] == str(fw), d
                assert g["kfw"] == str(kfw), d
        a = dwc.problem(2, 40, 40, 24, 6, fw, 1, (2, fw // 2))
        assert "generic" not in dwc.plan_describe(a, 2)
    p = dwc.problem(2, 40, 40, 24, 5, 32, 1, (2, 16))
    assert all(dwc.plan_describe(p, op).split()[1] == "generic" for op in (0, 2))


def test_no_kernel_uses_scratch():
    """Every kernel keeps its arrays in registers: the compiler's resource
    remarks (recorded by the build) show no per-lane scratch memory, which
    an array indexed past a loop exit or by a runtime value would need."""
    path = os.path.join(os.path.dirname(dwc.__file__), "kernel_resources.json")
    if not os.path.exists(path):
        pytest.skip("library not built")
    with open(path) as f:
        res = json.load(f)
    assert res and all("scratch" in v for v in res.values())
    assert {k: v["scratch"] for k, v in res.items() if v["scratch"]} == {}


def test_small_and_mid_filter_auto_rules():
    """AUTO (measured on MI355X): 16-bit and fp8 filters up to 5x5 stay on
    the vector kernels (fp8 filter gradients only up to 5 taps); wider ones
    take the packed matrix-core kernels; fp32 filters from 10x10 whose
    columns stop short of 13 take the fp32 matrix-core kernels at any width
    (the vector kernels would run them on their 13-wide body), 9x9 stays on
    the sweeps."""
    def fam(dt, fh, fw, op, n=64, h=28, c=256):
        p = dwc.problem(n, h, h, c, fh, fw, 1, (fh // 2, fw // 2), dtype=dt)
        return dwc.plan_describe(p, op).split()[1]
    for dt in (dwc.BF16, dwc.F16, dwc.FP8_E4M3):
        for fh, fw in ((1, 1), (3, 5), (5, 1), (2, 2), (4, 4)):
            for op in (0, 1):
                assert fam(dt, fh, fw, op) == "direct", (dt, fh, fw, op)
        for fh, fw in ((1, 7), (7, 3), (6, 6)):
            assert fam(dt, fh, fw, 0) == "mfma", (dt, fh, fw)
    for fh, fw in ((1, 1), (3, 5), (4, 4)):
        assert fam(dwc.BF16, fh, fw, 2) == "direct"
    assert fam(dwc.FP8_E4M3, 1, 5, 2) == "direct"
    assert fam(dwc.FP8_E4M3, 3, 5, 2) == "mfma"
    for h, c in ((56, 128), (28, 256), (14, 512), (7, 1024)):
        for op in (0, 1, 2):
            assert fam(dwc.F32, 11, 11, op, h=h, c=c) == "mfma", (h, op)
            assert fam(dwc.F32, 9, 9, op, h=h, c=c) == "sweep", (h, op)

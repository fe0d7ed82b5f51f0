"""Build libdwc.so in-tree: hipcc for gfx950, one object per translation unit.

Usage: ``python -m depthwise_convolution_dwc_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the library lands next to
this file as ``libdwc.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdwc.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Registers, occupancy and spills of every kernel, from the compiler's
# resource-usage remarks (the profile summaries read it)
RESOURCES = os.path.join(PKG, "kernel_resources.json")

# Every HIP translation unit is built without packed-fp32 instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", CSRC, "-I", INCLUDE,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", CSRC, "-I", INCLUDE]


def _units():
    """(compiler, source, object, extra flags) per translation unit."""
    u = []
    # the sweep kernels' row loops (lcm(F, 3) rows, 21 at 7x7) must unroll
    # completely, also with the fused prologue, so that every register-ring
    # index is a constant; LLVM's default size limit for that stops short
    for dt in (0, 1, 2, 3, 4):
        for pad in (0, 1):
            u.append(("hip", "inst_direct.hip", f"inst_direct_dt{dt}{'_pad' if pad else ''}.o",
                      [f"-DDWC_INST_DT={dt}", f"-DDWC_INST_PAD={pad}", "-mllvm",
                       "-pragma-unroll-threshold=30000"]))
    u.append(("hip", "inst_generic.hip", "inst_generic.o", []))
    # MFMA accumulators in VGPRs: with AGPR accumulators the compiler moves
    # them between registers on every filter-row iteration
    u.append(("hip", "inst_mfma.hip", "inst_mfma.o", ["-mllvm", "-amdgpu-mfma-vgpr-form"]))
    u.append(("hip", "inst_mfma8.hip", "inst_mfma8.o", ["-mllvm", "-amdgpu-mfma-vgpr-form"]))
    u.append(("hip", "inst_mfma_batch.hip", "inst_mfma_batch.o",
              ["-mllvm", "-amdgpu-mfma-vgpr-form"]))
    u.append(("hip", "inst_mfma_f32.hip", "inst_mfma_f32.o", ["-mllvm", "-amdgpu-mfma-vgpr-form"]))
    u.append(("hip", "inst_mfma_h4.hip", "inst_mfma_h4.o", ["-mllvm", "-amdgpu-mfma-vgpr-form"]))
    u.append(("hip", "dwc_api.cpp", "dwc_api.o", ["-x", "hip"]))
    u.append(("cxx", "dwc_plan.cpp", "dwc_plan.o", []))
    return u


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|Occupancy \[waves/SIMD\]|"
                     r"VGPRs Spill|SGPRs Spill|LDS Size \[bytes/block\]|"
                     r"ScratchSize \[bytes/lane\]):\s+(\S+)")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "Occupancy [waves/SIMD]": "waves_per_simd",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
           "LDS Size [bytes/block]": "lds_static", "ScratchSize [bytes/lane]": "scratch"}


def _resource_remarks(text):
    """{mangled kernel name: {field: int}} from -Rpass-analysis remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        k, v = m.group(1), m.group(2)
        if k == "Function Name":
            cur = out.setdefault(v, {})
        elif cur is not None:
            cur[_FIELDS[k]] = int(v)
    return out


def _compile(unit, verbose):
    kind, src, obj, extra = unit
    src_p = os.path.join(CSRC, src)
    obj_p = os.path.join(BUILD, obj)
    if kind == "hip":
        cmd = [HIPCC] + HIP_FLAGS + extra + ["-Rpass-analysis=kernel-resource-usage", "-c", src_p,
                                             "-o", obj_p]
    else:
        cmd = ["g++"] + CXX_FLAGS + extra + ["-c", src_p, "-o", obj_p]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    res = _resource_remarks(text)
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # the resource remarks are kept apart
    msgs = [ln for ln in text.splitlines()
            if "is not a recognized feature" not in ln and "kernel-resource-usage" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj_p, res


def _write_resources(res):
    """Demangled kernel names ('dwc::fwd_sweep<0, 7, 7, false, false>') to
    their registers, occupancy and spills."""
    names = sorted(res)
    demangled = names
    if shutil.which("c++filt"):
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
        if r.returncode == 0 and len(r.stdout.splitlines()) == len(names):
            demangled = r.stdout.splitlines()
    table = {}
    for mangled, dem in zip(names, demangled):
        key = dem.split("(")[0].replace("void ", "").strip()
        table[key] = res[mangled]
    tmp = RESOURCES + ".tmp"
    with open(tmp, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    os.replace(tmp, RESOURCES)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every translation unit and link libdwc.so; returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    units = _units()
    jobs = jobs or min(len(units), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(lambda u: _compile(u, verbose), units))
    objs = [o for o, _ in done]
    res = {}
    for _, r in done:
        res.update(r)
    _write_resources(res)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
           f"-Wl,--version-script={os.path.join(CSRC, 'libdwc.map')}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

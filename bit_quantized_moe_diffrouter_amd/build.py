"""Builds libqmoe.so (HIP for gfx950) in the package directory with hipcc.

Each kernel translation unit is compiled separately (in parallel), then all
objects are linked into one shared library.  A kernel that spills registers
to scratch memory fails the build.  The library is written to a
temporary name and renamed, so a concurrent reader never sees a half-written
file."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmoe.so")
ARCH = "gfx950"

HIP_SOURCES = ["qswitch.hip", "qmm_ws.hip", "qmm_tall.hip", "qswitch_unsorted.hip", "route.hip", "sort.hip", "ffblock.hip", "embed_t.hip"]
HOST_SOURCES = ["abi.cpp"]

# Packed-fp32 instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Matrix-core results in VGPRs (no accumulation-register round trips), except
# in the tall-tile kernel, whose one wave per SIMD keeps its sums in the
# accumulation registers.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_SOURCES = {"qmm_tall.hip"}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
                "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqmoe.so)")


# The compiler's per-kernel resource remarks: a kernel that spills registers
# to scratch memory fails the build (the hot loops are sized to fit).
RESOURCE_FLAGS = ["-Rpass-analysis=kernel-resource-usage"]
_REMARK = re.compile(r"remark:\s+(Function Name|SGPRs Spill|VGPRs Spill): (\S+)")


def spills(output: str):
    """(kernel, sgpr_spills, vgpr_spills) for every kernel in the remarks whose
    spill count is non-zero."""
    found, name, sgpr = [], None, 0
    for m in _REMARK.finditer(output):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            name, sgpr = val, 0
        elif key == "SGPRs Spill":
            sgpr = int(val)
        else:
            if sgpr or int(val):
                found.append((name, sgpr, int(val)))
    return found


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    bad = spills(out)
    if bad:
        raise RuntimeError("register spills in " + ", ".join(f"{n} (SGPR {s}, VGPR {v})" for n, s, v in bad))
    if verbose:
        shown = "\n".join(l for l in out.splitlines() if "remark:" not in l)
        if shown.strip():
            print(shown)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libqmoe.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        form = [] if src in AGPR_SOURCES else VGPR_FORM
        jobs.append([hipcc, f"--offload-arch={ARCH}", *COMMON_FLAGS, *DEVICE_FLAGS, *form, *RESOURCE_FLAGS, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, src.replace(".cpp", ".o"))
        jobs.append([hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""The C ABI's host code (argument validation, size arithmetic, error
strings: csrc/abi.cpp) built with AddressSanitizer and UndefinedBehavior-
Sanitizer, then driven by the host-side ABI and binding tests in a child
process.  Only the host translation unit is instrumented (with g++); the
kernel objects are linked unchanged and never launched, since every call
in those tests is rejected or sized before anything reaches a device.  Any
out-of-bounds access, overflow or other undefined behaviour aborts the child,
which fails this test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from _util import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_quantized_moe_diffrouter_amd")

RUNNER = r"""
import sys
sys.path[:0] = [{tests!r}, {root!r}]
import bit_quantized_moe_diffrouter_amd as q
q.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main([{t1!r}, {t2!r}, "-q", "-p", "no:cacheprovider", "-k", "not plain_c"]))
"""


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("the sanitizer runtimes are not installed")
    ensure_built()
    kernels = [o for o in glob.glob(os.path.join(PKG, "_build", "*.o")) if os.path.basename(o) != "abi.o"]
    assert kernels, "the kernel objects are missing"
    obj, lib = tmp_path / "abi_san.o", tmp_path / "libqmoe_san.so"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(PKG, "csrc", "abi.cpp"), "-o", str(obj)],
                   check=True, capture_output=True, timeout=300)
    subprocess.run(["g++", "-shared", *san, "-o", str(lib), str(obj), *kernels, "-L", "/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True, timeout=300)
    script = RUNNER.format(tests=os.path.join(ROOT, "tests"), root=ROOT, lib=str(lib),
                           t1=os.path.join(ROOT, "tests", "test_abi_host.py"),
                           t2=os.path.join(ROOT, "tests", "test_binding_checks.py"))
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=600,
                         cwd=str(tmp_path))
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "passed" in run.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out

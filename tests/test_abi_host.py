"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, sizes its workspaces, and rejects bad
arguments with the documented codes before anything reaches the device."""
import ctypes
import os
import re

import pytest

from _util import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3
A16 = 0x100000  # a 16-byte aligned fake device address: validation never dereferences it


@pytest.fixture(scope="module")
def L():
    return ensure_built()


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) >= {"moe_route", "moe_sort", "qswitch_gate_up_geglu", "qswitch_down_combine",
                          "qlinear", "qmoe_last_error", "ff_prenorm", "qlinear_geglu", "ff_combine",
                          "qswitch_gate_up_geglu_unsorted", "qswitch_down_combine_unsorted",
                          "qlinear_softcap", "softmax_rows_bf16", "embed_matmul_t", "qmoe_tile_weight_t"}
    for n in names:
        assert hasattr(L, n), f"{n} is declared in qmoe.h but not exported"


def qw(experts, rows, inp, bits=4, group=64, w=A16, s=A16, b=A16, layout=0, split=0):
    import bit_quantized_moe_diffrouter_amd as q
    return q.QWeightDesc(w, s, b, experts, rows, inp, bits, group, layout, split)


def err(L):
    return L.qmoe_last_error().decode()


def route(L, T=16, H=256, E=8, k=2, x=A16, ws=A16, ws_bytes=1 << 30, **kw):
    d = qw(1, E, H, **kw)
    return L.moe_route(x, T, H, A16, 1e-6, ctypes.byref(d), A16, None, k, A16, A16, None, ws, ws_bytes, None)


def test_route_validation(L):
    assert route(L, T=0, x=None, ws=None, ws_bytes=0) == 0  # T = 0 is a no-op
    assert route(L, H=100) == INVALID and "H=100" in err(L)
    assert route(L, T=-1) == INVALID
    assert route(L, E=300) == UNSUPPORTED
    assert route(L, k=0) == UNSUPPORTED
    assert route(L, k=9, E=8) == UNSUPPORTED
    assert route(L, k=17, E=64) == UNSUPPORTED
    assert route(L, bits=8) == UNSUPPORTED and "bits" in err(L)
    assert route(L, group=32) == UNSUPPORTED
    assert route(L, x=None) == INVALID and "null" in err(L)
    assert route(L, x=A16 + 2) == INVALID and "aligned" in err(L)
    assert route(L, ws_bytes=16) == WORKSPACE
    assert route(L, ws=None) == WORKSPACE
    d = qw(1, 8, 128)  # in != H
    assert L.moe_route(A16, 16, 256, A16, 1e-6, ctypes.byref(d), A16, None, 2, A16, A16, None, A16, 1 << 30,
                       None) == INVALID


def test_sort_validation(L):
    assert L.moe_sort(None, 0, 2, 8, None, None, None, 0, None) == 0
    assert L.moe_sort(A16, -1, 2, 8, A16, A16, None, 0, None) == INVALID
    assert L.moe_sort(A16, 4, 0, 8, A16, A16, None, 0, None) == INVALID
    assert L.moe_sort(A16, 4, 2, 0, A16, A16, None, 0, None) == UNSUPPORTED
    assert L.moe_sort(A16, 4, 2, 257, A16, A16, None, 0, None) == UNSUPPORTED
    assert L.moe_sort(A16, 1 << 22, 8, 8, A16, A16, None, 0, None) == UNSUPPORTED
    assert L.moe_sort(None, 4, 2, 8, A16, A16, None, 0, None) == INVALID
    assert L.moe_sort(A16, 4, 2, 8, A16 + 2, A16, None, 0, None) == INVALID
    assert L.moe_sort(A16, 4, 2, 8, A16, A16, A16 + 2, 64, None) == INVALID   # misaligned workspace


def test_sort_workspace_sizes(L):
    # 0 below 8192 assignments; above, one (E+1)-int histogram per slice, slices
    # a multiple of 1024 assignments and at most 256 of them
    assert L.moe_sort_workspace(256, 8, 128) == 0
    assert L.moe_sort_workspace(1023, 8, 128) == 0
    assert L.moe_sort_workspace(1024, 8, 128) == 8 * 129 * 4
    assert L.moe_sort_workspace(4096, 8, 128) == 32 * 129 * 4
    assert L.moe_sort_workspace(18750, 16, 256) == 147 * 257 * 4       # slices of 2048
    assert L.moe_sort_workspace(1 << 21, 8, 256) == 256 * 257 * 4      # 2^24: slices of 65536
    assert L.moe_sort_workspace(0, 8, 128) == 0
    assert L.moe_sort_workspace(1 << 22, 8, 128) == 0                  # above the limit


def gate_up(L, T=16, H=256, I=128, k=2, E=8, rows=None, inp=None, x=A16, mid=A16, mid_bytes=1 << 30, layout=1,
            split=None, **kw):
    d = qw(E, 2 * I if rows is None else rows, H if inp is None else inp, layout=layout,
           split=I if split is None else split, **kw)
    return L.qswitch_gate_up_geglu(x, T, H, ctypes.byref(d), I, k, A16, A16, mid, mid_bytes, None)


def test_gate_up_validation(L):
    assert gate_up(L, T=0) == 0
    assert gate_up(L, I=100) == INVALID
    assert gate_up(L, H=96) == INVALID
    assert gate_up(L, k=0) == UNSUPPORTED
    assert gate_up(L, rows=100) == INVALID
    assert gate_up(L, inp=512) == INVALID
    assert gate_up(L, E=0) == UNSUPPORTED
    assert gate_up(L, group=128) == UNSUPPORTED
    assert gate_up(L, mid=None) == INVALID
    assert gate_up(L, mid=A16 + 8) == INVALID
    assert gate_up(L, x=None) == INVALID
    assert gate_up(L, x=A16 + 2) == INVALID
    assert gate_up(L, layout=0) == INVALID and "qmoe_tile_weight" in err(L)
    assert gate_up(L, split=0) == INVALID and "split" in err(L)
    need_mid = L.qswitch_mid_bytes(16, 2, 128, 8)
    assert gate_up(L, mid_bytes=need_mid - 1) == INVALID and "mid" in err(L)


def test_activation_tile_sizes(L):
    # (ceil(A / 16) + min(E, A)) tiles of (C / 64) blocks of 2048 bytes
    assert L.qswitch_mid_bytes(256, 8, 704, 128) == (128 + 128) * 11 * 2048
    assert L.qswitch_mid_bytes(256, 8, 2816, 128) == (128 + 128) * 44 * 2048
    assert L.qswitch_mid_bytes(4096, 8, 704, 128) == (2048 + 128) * 11 * 2048
    assert L.qswitch_mid_bytes(3, 1, 64, 8) == (1 + 3) * 1 * 2048  # min(E, A) partial tiles at most
    assert L.qswitch_mid_bytes(37, 3, 192, 12) == (7 + 12) * 3 * 2048
    assert L.qswitch_mid_bytes(0, 8, 704, 128) == 0
    assert L.qswitch_mid_bytes(16, 2, 100, 8) == 0
    assert L.qswitch_mid_bytes(16, 2, 96, 8) == 0


def down(L, T=16, H=256, I=128, k=2, E=8, ws=A16, ws_bytes=1 << 30, y=A16, layout=1, **kw):
    d = qw(E, H, I, layout=layout, **kw)
    return L.qswitch_down_combine(A16, T, k, I, ctypes.byref(d), H, A16, A16, A16, y, ws, ws_bytes, 1, None)


def test_down_validation(L):
    assert down(L, T=0, ws=None, ws_bytes=0) == 0
    assert down(L, H=200) == INVALID
    assert down(L, I=32) == INVALID
    assert down(L, ws_bytes=100) == WORKSPACE and "workspace" in err(L)
    assert down(L, ws=None) == WORKSPACE
    assert down(L, y=None) == INVALID
    assert down(L, bits=3) == UNSUPPORTED
    assert down(L, layout=0) == INVALID
    assert down(L, split=64) == INVALID
    assert L.qswitch_down_combine_workspace(256, 8, 2816, 1) == 256 * 8 * 2816 * 2  # bf16 down rows


def test_qlinear_validation(L):
    d = qw(1, 1152, 1152, layout=1)
    assert L.qlinear(None, 0, ctypes.byref(d), None, None) == 0
    assert L.qlinear(A16, -5, ctypes.byref(d), A16, None) == INVALID
    bad = qw(1, 1150, 1152, layout=1)
    assert L.qlinear(A16, 8, ctypes.byref(bad), A16, None) == INVALID
    bad = qw(1, 1152, 1000, layout=1)
    assert L.qlinear(A16, 8, ctypes.byref(bad), A16, None) == INVALID
    bad = qw(2, 1152, 1152, layout=1)
    assert L.qlinear(A16, 8, ctypes.byref(bad), A16, None) == INVALID
    bad = qw(1, 1152, 1152, layout=0)
    assert L.qlinear(A16, 8, ctypes.byref(bad), A16, None) == INVALID
    assert L.qlinear(A16, 8, None, A16, None) == INVALID


def test_qlinear_softcap_validation(L):
    f = ctypes.c_float
    d = qw(1, 4096, 256, layout=1)
    assert L.qlinear_softcap(None, 0, ctypes.byref(d), f(30.0), None, None) == 0
    assert L.qlinear_softcap(A16, -1, ctypes.byref(d), f(30.0), A16, None) == INVALID
    for cap in (0.0, -30.0, float("inf"), float("nan")):
        assert L.qlinear_softcap(A16, 4, ctypes.byref(d), f(cap), A16, None) == INVALID
    assert "cap" in err(L)
    assert L.qlinear_softcap(A16, 4, ctypes.byref(qw(1, 4100, 256, layout=1)), f(30.0), A16, None) == INVALID
    assert L.qlinear_softcap(A16, 4, ctypes.byref(qw(1, 4096, 256, layout=1, split=2048)), f(30.0), A16,
                             None) == INVALID
    assert L.qlinear_softcap(A16, 4, ctypes.byref(d), f(30.0), A16 + 4, None) == INVALID


def test_embed_matmul_t_validation(L):
    f = ctypes.c_float
    assert L.qmoe_tiled_weight_t_bytes(262144, 2816) == 44 * 8192 * 1152
    assert L.qmoe_tiled_weight_t_bytes(100, 2816) == 0 and L.qmoe_tiled_weight_t_bytes(256, 100) == 0
    ws = L.embed_matmul_t_workspace(16, 1024, 256)
    assert ws > 0 and ws % (16 * 256 * 4) == 0
    d = qw(1, 1024, 256, layout=2)
    e = lambda Lr=16, W=d, p=A16, sc=1.0, o=A16, w=A16, n=ws: L.embed_matmul_t(p, Lr, ctypes.byref(W), f(sc), o, w, n,
                                                                             None)
    assert e(Lr=0, p=None, o=None) == 0
    assert e(Lr=-1) == INVALID
    assert e(W=qw(1, 1000, 256, layout=2)) == INVALID      # rows % 32
    assert e(W=qw(1, 1024, 256, layout=1)) == INVALID      # not the untransposed tiling
    assert e(W=qw(2, 1024, 256, layout=2)) == INVALID      # one table
    assert e(sc=float("nan")) == INVALID
    assert e(o=A16 + 2) == INVALID
    assert e(n=ws - 1) == WORKSPACE
    assert L.softmax_rows_bf16(A16, 4, 1022, A16, None) == INVALID
    assert L.softmax_rows_bf16(None, 4, 1024, A16, None) == INVALID
    assert L.softmax_rows_bf16(None, 0, 1024, None, None) == 0
    src = qw(1, 1024, 256)
    assert L.qmoe_tile_weight_t(ctypes.byref(src), A16, L.qmoe_tiled_weight_t_bytes(1024, 256) - 1, None) == INVALID
    assert L.qmoe_tile_weight_t(ctypes.byref(qw(1, 1024, 256, layout=1)), A16, 1 << 30, None) == INVALID


def test_qlinear_geglu_validation(L):
    d = qw(1, 2 * 192, 256, layout=1, split=192)
    assert L.qlinear_geglu(None, 0, ctypes.byref(d), None, None) == 0
    assert L.qlinear_geglu(A16, -1, ctypes.byref(d), A16, None) == INVALID
    for bad in (qw(1, 2 * 192, 256, layout=1, split=0),      # not tiled as a fused pair
                qw(1, 2 * 192, 256, layout=1, split=128),    # rows != 2 * split
                qw(1, 2 * 72, 256, layout=1, split=72),      # split not a multiple of 16
                qw(1, 2 * 192, 200, layout=1, split=192),    # K not a multiple of 64
                qw(2, 2 * 192, 256, layout=1, split=192),    # not dense
                qw(1, 2 * 192, 256, layout=0, split=192)):   # row-major codes
        assert L.qlinear_geglu(A16, 8, ctypes.byref(bad), A16, None) == INVALID, err(L)
    assert L.qlinear_geglu(A16 + 8, 8, ctypes.byref(d), A16, None) == INVALID
    assert "aligned" in err(L)
    assert L.qlinear_geglu(A16, 8, ctypes.byref(d), None, None) == INVALID
    assert L.qlinear_geglu(A16, 8, ctypes.byref(qw(1, 384, 256, bits=8, layout=1, split=192)), A16,
                           None) == UNSUPPORTED


def test_ff_norm_validation(L):
    f = ctypes.c_float
    pre = lambda T=4, H=256, h=A16, wa=A16, wb=A16, eps=1e-6, xa=A16, xb=A16: L.ff_prenorm(
        h, T, H, wa, wb, f(eps), xa, xb, None)
    assert pre(T=0, h=None) == 0
    assert pre(T=-1) == INVALID
    assert pre(H=252) == INVALID
    assert "multiple of 8" in err(L)
    assert pre(eps=-1.0) == INVALID
    assert pre(eps=float("nan")) == INVALID
    assert pre(h=None) == INVALID
    assert pre(wb=A16 + 2) == INVALID
    assert pre(xa=None) == INVALID

    comb = lambda T=4, H=256, h=A16, d=A16, m=A16, w1=A16, w2=A16, w=A16, eps=1e-6, out=A16: L.ff_combine(
        h, d, m, T, H, w1, w2, w, f(eps), f(1.0), out, None)
    assert comb(T=0, h=None, out=None) == 0
    assert comb(T=-3) == INVALID
    assert comb(H=0) == INVALID
    assert comb(eps=float("inf")) == INVALID
    assert comb(m=None) == INVALID
    assert comb(w2=A16 + 4) == INVALID
    assert comb(out=None) == INVALID


def test_unsorted_workspace_sizes(L):
    # T=1, k=8, canvas: gate_up plan 1 group per wave, 11 workgroups per (assignment, block)
    # T=1: one group per wave; gate_up 11 workgroups per (assignment, block), down 3
    assert L.qswitch_unsorted_workspace(1, 8, 2816, 704) == max(8 * 11 * 11, 8 * 22 * 3) * 128 * 4
    assert L.qswitch_unsorted_workspace(512, 8, 2816, 704) > 0
    assert L.qswitch_unsorted_workspace(513, 8, 2816, 704) == 0      # T*k above 4096
    assert L.qswitch_unsorted_workspace(1, 8, 2800, 704) == 0        # H % 64
    assert L.qswitch_unsorted_workspace(0, 8, 2816, 704) == 0


def test_unsorted_validation(L):
    ws = L.qswitch_unsorted_workspace(2, 4, 256, 128)
    gu = qw(8, 256, 256, layout=1, split=128)
    dn = qw(8, 256, 128, layout=1)
    g = lambda T=2, H=256, I=128, k=4, d=gu, x=A16, idx=A16, mid=A16, w=A16, n=ws: \
        L.qswitch_gate_up_geglu_unsorted(x, T, H, ctypes.byref(d), I, k, idx, mid, w, n, None)
    dcall = lambda T=2, H=256, I=128, k=4, d=dn, mid=A16, idx=A16, wt=A16, y=A16, w=A16, n=ws: \
        L.qswitch_down_combine_unsorted(mid, T, k, I, ctypes.byref(d), H, idx, wt, y, w, n, None)
    assert g(T=0, x=None, mid=None) == 0
    assert g(T=-1) == INVALID
    assert g(H=200) == INVALID
    assert g(k=17) == UNSUPPORTED
    assert g(T=1025) == UNSUPPORTED
    assert "sorted calls" in err(L)
    assert g(d=qw(8, 256, 256, layout=1, split=0)) == INVALID       # not tiled as a fused pair
    assert g(d=qw(300, 256, 256, layout=1, split=128)) == UNSUPPORTED
    assert g(idx=None) == INVALID
    assert g(w=A16 + 8) == INVALID                                   # workspace not 16-byte aligned
    assert g(n=ws - 1) == WORKSPACE
    assert g(mid=None) == INVALID
    assert dcall(T=0, mid=None, y=None) == 0
    assert dcall(d=qw(8, 256, 128, layout=1, split=64)) == INVALID
    assert dcall(wt=None) == INVALID
    assert dcall(y=A16 + 8) == INVALID
    assert dcall(n=0) == WORKSPACE


def test_route_rejects_tiled_proj(L):
    d = qw(1, 8, 256, layout=1)
    assert L.moe_route(A16, 16, 256, A16, 1e-6, ctypes.byref(d), A16, None, 2, A16, A16, None, A16, 1 << 30,
                       None) == INVALID


def test_tile_weight_sizes_and_validation(L):
    # units of 4608 bytes per (expert, 128-row block, 64-wide group)
    assert L.qmoe_tiled_weight_bytes(128, 1408, 2816, 704) == 128 * 11 * 44 * 4608
    assert L.qmoe_tiled_weight_bytes(128, 2816, 704, 0) == 128 * 22 * 11 * 4608
    assert L.qmoe_tiled_weight_bytes(1, 1152, 1152, 0) == 1 * 9 * 18 * 4608
    assert L.qmoe_tiled_weight_bytes(1, 48, 192, 0) == 1 * 1 * 3 * 4608  # rows padded to a block
    assert L.qmoe_tiled_weight_bytes(8, 256, 100, 0) == 0
    assert L.qmoe_tiled_weight_bytes(8, 200, 256, 100) == 0  # split must be rows / 2, a multiple of 16
    # a fused pair whose width is a multiple of 16 only (the vision MLP's 4304): 68 blocks of 64 columns
    assert L.qmoe_tiled_weight_bytes(1, 2 * 4304, 1152, 4304) == 68 * 18 * 4608
    src = qw(8, 256, 256)
    need = L.qmoe_tiled_weight_bytes(8, 256, 256, 128)
    assert L.qmoe_tile_weight(ctypes.byref(src), 128, A16, need - 1, None) == INVALID
    assert L.qmoe_tile_weight(ctypes.byref(src), 100, A16, 1 << 30, None) == INVALID
    assert L.qmoe_tile_weight(ctypes.byref(src), 128, None, 1 << 30, None) == INVALID
    tiled_src = qw(8, 256, 256, layout=1)
    assert L.qmoe_tile_weight(ctypes.byref(tiled_src), 0, A16, 1 << 30, None) == INVALID
    assert L.qmoe_tile_weight(None, 0, A16, 1 << 30, None) == INVALID


def test_route_workspace_size(L):
    # 16-token tiles; the k-range split keeps about 256 workgroups busy, and
    # is at least 4 (at most the number of groups)
    assert L.moe_route_workspace(256, 2816, 128) == 16 * 256 * 129 * 4
    assert L.moe_route_workspace(4096, 2816, 128) == 4 * 4096 * 129 * 4
    assert L.moe_route_workspace(16, 256, 8) == 4 * 16 * 9 * 4
    assert L.moe_route_workspace(0, 256, 8) == 0
    assert L.moe_route_workspace(1, 2816, 128) == 16 * 1 * 129 * 4   # at most 16 parts


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "qmoe.h"

int main(void) {
    qmoe_qweight w;
    memset(&w, 0, sizeof w);
    if (qswitch_mid_bytes(256, 8, 704, 128) != (size_t)(128 + 128) * 11 * 2048) return 2;
    if (moe_route_workspace(0, 256, 8) != 0) return 3;
    if (qlinear(NULL, 4, &w, NULL, 0) != QMOE_ERR_INVALID) return 4;
    if (strstr(qmoe_last_error(), "qlinear") == NULL) return 5;
    puts(qmoe_last_error());
    return 0;
}
"""


def test_header_is_plain_c_and_links(L, tmp_path):
    """A C11 program includes the header, links the library and reaches its
    validation: the boundary needs no C++ or torch on the caller's side."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    lib_dir = os.path.dirname(L._name)
    src, exe = tmp_path / "caller.c", tmp_path / "caller"
    src.write_text(C_CALLER)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o", str(exe),
           "-L", lib_dir, "-lqmoe", f"-Wl,-rpath,{lib_dir}"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=120)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert "qlinear" in run.stdout


def test_build_rejects_register_spills():
    """The build reads the compiler's per-kernel resource remarks and fails on
    any kernel that spills registers to scratch memory."""
    from bit_quantized_moe_diffrouter_amd import build
    tail = " [-Rpass-analysis=kernel-resource-usage]"
    remarks = "\n".join(f"x.hip:1:1: remark: {l}{tail}" for l in [
        "Function Name: _ZN4qmoe3fooEv", "    SGPRs Spill: 0", "    VGPRs Spill: 12",
        "Function Name: _ZN4qmoe3barEv", "    SGPRs Spill: 0", "    VGPRs Spill: 0",
        "Function Name: _ZN4qmoe3bazEv", "    SGPRs Spill: 3", "    VGPRs Spill: 0"])
    assert build.spills(remarks) == [("_ZN4qmoe3fooEv", 0, 12), ("_ZN4qmoe3bazEv", 3, 0)]
    assert "-Rpass-analysis=kernel-resource-usage" in build.RESOURCE_FLAGS

"""4-bit group-quantized mixture-of-experts layer for AMD MI355X (gfx950).

Thin Python binding of ``libqmoe.so`` (C ABI in ``include/qmoe.h``): argument
marshalling only.  Every step of the layer runs in the library's HIP kernels;
PyTorch supplies device memory and the current stream.  If the library has not
been built, every call raises -- there is no fallback path.

The layer (diffusion-gemma model.ts page of the "@mlx-bun/inference" diff:
DiffRouter, DiffExperts, DiffDecoderLayer.forwardWith):

    indices, weights = moe_route(x_router, ...)           # DiffRouter
    offsets, sorted  = moe_sort(indices, E)               # token-by-expert sort
    mid = qswitch_gate_up_geglu(x_expert, gate_up, ...)   # gate_up, split, GeGLU
    y   = qswitch_down_combine(mid, down, weights, ...)   # down, weighted sum over k
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

__all__ = [
    "QMoEError", "QuantWeight", "TiledWeight", "MoEParams", "lib", "library_path",
    "moe_route", "moe_route_workspace", "moe_sort", "moe_sort_workspace", "qswitch_mid_bytes",
    "qswitch_gate_up_geglu", "device_status",
    "qswitch_down_combine", "qswitch_down_combine_workspace", "qswitch_down_combine_noalloc", "qlinear", "moe_layer",
    "ff_prenorm", "qlinear_geglu", "ff_combine", "FFParams", "ff_block", "qlinear_softcap",
    "TiledTWeight", "softmax_rows_bf16", "embed_matmul_t", "self_condition_embed",
    "qswitch_unsorted_workspace", "unsorted_workspace", "qswitch_gate_up_geglu_unsorted",
    "qswitch_down_combine_unsorted", "moe_layer_unsorted",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

QMOE_OK, QMOE_ERR_INVALID, QMOE_ERR_UNSUPPORTED, QMOE_ERR_WORKSPACE, QMOE_ERR_HIP = 0, -1, -2, -3, -4


class QMoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class QWeightDesc(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("biases", ctypes.c_void_p),
        ("experts", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("in_", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("split", ctypes.c_int32),
    ]

LAYOUT_ROWS, LAYOUT_TILED = 0, 1


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_QP = ctypes.POINTER(QWeightDesc)

_SIGNATURES = {
    "qmoe_last_error": (ctypes.c_char_p, []),
    "moe_route_workspace": (_SZ, [_I, _I, _I]),
    "moe_route": (ctypes.c_int, [_P, _I, _I, _P, ctypes.c_float, _QP, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_sort_workspace": (_SZ, [_I, _I, _I]),
    "moe_sort": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "qswitch_mid_bytes": (_SZ, [_I, _I, _I, _I]),
    "qswitch_gate_up_geglu": (ctypes.c_int, [_P, _I, _I, _QP, _I, _I, _P, _P, _P, _SZ, _P]),
    "qmoe_device_status": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32), _I]),
    "qswitch_down_combine_workspace": (_SZ, [_I, _I, _I, _I]),
    "qswitch_down_combine": (ctypes.c_int, [_P, _I, _I, _I, _QP, _I, _P, _P, _P, _P, _P, _SZ, _I, _P]),
    "qswitch_down_combine_noalloc": (ctypes.c_int, [_P, _I, _I, _I, _QP, _I, _P, _P, _P, _P, _I, _P]),
    "qlinear": (ctypes.c_int, [_P, _I, _QP, _P, _P]),
    "qlinear_geglu": (ctypes.c_int, [_P, _I, _QP, _P, _P]),
    "qlinear_softcap": (ctypes.c_int, [_P, _I, _QP, ctypes.c_float, _P, _P]),
    "qmoe_tiled_weight_t_bytes": (_SZ, [_I, _I]),
    "qmoe_tile_weight_t": (ctypes.c_int, [_QP, _P, _SZ, _P]),
    "softmax_rows_bf16": (ctypes.c_int, [_P, _I, _I, _P, _P]),
    "embed_matmul_t_workspace": (_SZ, [_I, _I, _I]),
    "embed_matmul_t": (ctypes.c_int, [_P, _I, _QP, ctypes.c_float, _P, _P, _SZ, _P]),
    "qswitch_unsorted_workspace": (_SZ, [_I, _I, _I, _I]),
    "qswitch_gate_up_geglu_unsorted": (ctypes.c_int, [_P, _I, _I, _QP, _I, _I, _P, _P, _P, _SZ, _P]),
    "qswitch_down_combine_unsorted": (ctypes.c_int, [_P, _I, _I, _I, _QP, _I, _P, _P, _P, _P, _SZ, _P]),
    "ff_prenorm": (ctypes.c_int, [_P, _I, _I, _P, _P, ctypes.c_float, _P, _P, _P]),
    "ff_combine": (ctypes.c_int, [_P, _P, _P, _I, _I, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P]),
    "qmoe_tiled_weight_bytes": (_SZ, [_I, _I, _I, _I]),
    "qmoe_tile_weight": (ctypes.c_int, [_QP, _I, _P, _SZ, _P]),
}

_lib = None


def library_path() -> str:
    return LIB_PATH


def lib():
    """The loaded libqmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m bit_quantized_moe_diffrouter_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != QMOE_OK:
        raise QMoEError(rc, lib().qmoe_last_error().decode())


def _dptr(t: torch.Tensor) -> int:
    """Device address of a tensor handed to the library (host tensors refused)."""
    if not t.is_cuda:
        raise ValueError(f"a {tuple(t.shape)} {t.dtype} argument must be a device tensor")
    return t.data_ptr()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(_dptr(t))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, elem: int, shape=None):
    """Checks a tensor handed to the library: element size, shape and layout
    (the C calls take bare pointers, so this is the only size check some
    arguments get).  Raises before anything is launched; residence on the
    device is checked when the pointer is taken (_dptr)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.element_size() != elem:
        raise ValueError(f"{name}: element size {t.element_size()}, expected {elem}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _need_opt(t: Optional[torch.Tensor], name: str, elem: int, shape=None):
    if t is not None:
        _need(t, name, elem, shape)


def _same(a: int, b: int, what: str):
    if int(a) != int(b):
        raise ValueError(f"{what}: {a} != {b}")


@dataclass
class QuantWeight:
    """Device-resident 4-bit weight: codes uint32 ``[E?, rows, in/8]``, bf16
    scales and biases ``[E?, rows, in/64]`` (as torch.uint16 or torch.bfloat16)."""

    w: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor

    @property
    def experts(self) -> int:
        return 1 if self.w.dim() == 2 else int(self.w.shape[0])

    @property
    def rows(self) -> int:
        return int(self.w.shape[-2])

    @property
    def in_features(self) -> int:
        return int(self.w.shape[-1]) * 8

    def desc(self) -> QWeightDesc:
        _need(self.w, "weight codes", 4)
        _need(self.scales, "weight scales", 2)
        _need(self.biases, "weight biases", 2)
        g = self.in_features // 64
        lead = tuple(self.w.shape[:-1])
        if tuple(self.scales.shape) != lead + (g,) or tuple(self.biases.shape) != lead + (g,):
            raise ValueError("scales/biases shape does not match the codes")
        return QWeightDesc(_dptr(self.w), _dptr(self.scales), _dptr(self.biases),
                           self.experts, self.rows, self.in_features, 4, 64, LAYOUT_ROWS, 0)

    @classmethod
    def from_numpy(cls, w, scales, biases, device="cuda") -> "QuantWeight":
        return cls(torch.from_numpy(w).to(device), torch.from_numpy(scales).to(device),
                   torch.from_numpy(biases).to(device))

    def tiled_t(self) -> "TiledTWeight":
        """The re-laid copy the untransposed product reads (qmoe_tile_weight_t)."""
        n = int(lib().qmoe_tiled_weight_t_bytes(self.rows, self.in_features))
        if n == 0 or self.experts != 1 or self.w.dim() != 2:
            raise ValueError(f"cannot tile a [{self.rows}, {self.in_features}] table for the untransposed product")
        buf = torch.empty(n, dtype=torch.uint8, device=self.w.device)
        d = self.desc()
        _check(lib().qmoe_tile_weight_t(ctypes.byref(d), _ptr(buf), n, _stream()))
        return TiledTWeight(buf, self.rows, self.in_features)

    def tiled(self, split: int = 0) -> "TiledWeight":
        """The tiled copy the switch linears and qlinear read (qmoe_tile_weight)."""
        n = int(lib().qmoe_tiled_weight_bytes(self.experts, self.rows, self.in_features, split))
        if n == 0:
            raise ValueError(f"cannot tile a [{self.experts}, {self.rows}, {self.in_features}] weight "
                             f"with split={split}")
        buf = torch.empty(n, dtype=torch.uint8, device=self.w.device)
        d = self.desc()
        _check(lib().qmoe_tile_weight(ctypes.byref(d), int(split), _ptr(buf), n, _stream()))
        return TiledWeight(buf, self.experts, self.rows, self.in_features, int(split))


@dataclass
class TiledWeight:
    """A weight in the tiled layout (one device byte buffer; see qmoe_tile_weight)."""

    buf: torch.Tensor
    experts: int
    rows: int
    in_features: int
    split: int = 0

    def desc(self) -> QWeightDesc:
        _need(self.buf, "tiled weight", 1)
        return QWeightDesc(_dptr(self.buf), None, None, self.experts, self.rows, self.in_features, 4, 64,
                           LAYOUT_TILED, self.split)


def moe_route_workspace(T: int, H: int, E: int) -> int:
    return int(lib().moe_route_workspace(T, H, E))


def moe_route(x_router: torch.Tensor, norm_scale: torch.Tensor, eps: float, proj: QuantWeight,
              per_expert_scale: torch.Tensor, k: int, logit_bias: Optional[torch.Tensor] = None,
              logits_out: Optional[torch.Tensor] = None, indices: Optional[torch.Tensor] = None,
              weights: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """DiffRouter: returns (indices int32 [T, k], weights fp32 [T, k])."""
    _need(x_router, "x_router", 2)
    T, H = (int(v) for v in x_router.shape)
    E = proj.rows
    dev = x_router.device
    _same(proj.in_features, H, "router weight in_features vs x_router.shape[1]")
    _need(norm_scale, "norm_scale", 2, (H,))
    _need(per_expert_scale, "per_expert_scale", 2, (E,))
    _need_opt(logit_bias, "logit_bias (fp32)", 4, (E,))
    _need_opt(logits_out, "logits_out (fp32)", 4, (T, E))
    _need_opt(indices, "indices", 4, (T, k))
    _need_opt(weights, "weights (fp32)", 4, (T, k))
    _need_opt(workspace, "workspace", 1)
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    need = moe_route_workspace(T, H, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = proj.desc()
    _check(lib().moe_route(_ptr(x_router), T, H, _ptr(norm_scale), float(eps), ctypes.byref(d),
                           _ptr(per_expert_scale), _ptr(logit_bias), k, _ptr(indices), _ptr(weights),
                           _ptr(logits_out), _ptr(workspace), ws_bytes, _stream()))
    return indices, weights


def moe_sort_workspace(T: int, k: int, E: int) -> int:
    """Bytes of the sort's workspace (0 below 8192 assignments)."""
    return int(lib().moe_sort_workspace(T, k, E))


def moe_sort(indices: torch.Tensor, E: int, expert_offsets: Optional[torch.Tensor] = None,
             sorted_assign: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             slices: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Token-by-expert sort: returns (expert_offsets int32 [E+1], sorted_assign int32 [T*k]).
    A workspace is allocated when none is given and the input is large enough
    for the slice sort; slices=False passes none, so one workgroup sorts."""
    _need(indices, "indices", 4)
    T, k = (int(v) for v in indices.shape)
    _need_opt(expert_offsets, "expert_offsets", 4, (E + 1,))
    _need_opt(sorted_assign, "sorted_assign", 4, (T * k,))
    _need_opt(workspace, "workspace", 1)
    dev = indices.device
    if expert_offsets is None:
        expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if sorted_assign is None:
        sorted_assign = torch.empty(T * k, dtype=torch.int32, device=dev)
    if not slices:
        workspace = None
    elif workspace is None:
        need = moe_sort_workspace(T, k, E)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_sort(_ptr(indices), T, k, E, _ptr(expert_offsets), _ptr(sorted_assign),
                          None if workspace is None else _ptr(workspace), _nbytes(workspace), _stream()))
    return expert_offsets, sorted_assign


def qswitch_mid_bytes(T: int, k: int, C: int, E: int) -> int:
    """Bytes of an activation-tile buffer of C columns (the layout of mid, see qmoe.h)."""
    return int(lib().qswitch_mid_bytes(T, k, C, E))


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def qswitch_gate_up_geglu(x_expert: torch.Tensor, gate_up: "TiledWeight", I: int, k: int,
                          expert_offsets: torch.Tensor, sorted_assign: torch.Tensor,
                          mid: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gate_up switch linear + split + GeGLU: returns mid, a uint8 buffer of activation tiles
    (I columns, the sorted rows of each expert in 16-row tiles; layout in qmoe.h)."""
    _need(x_expert, "x_expert", 2)
    T, H = (int(v) for v in x_expert.shape)
    E = gate_up.experts
    _same(gate_up.in_features, H, "gate_up in_features vs x_expert.shape[1]")
    _same(gate_up.rows, 2 * I, "gate_up rows vs 2 * I")
    _need(expert_offsets, "expert_offsets", 4, (E + 1,))
    _need(sorted_assign, "sorted_assign", 4, (T * k,))
    _need_opt(mid, "mid", 1)
    if mid is None:
        mid = torch.empty(max(1, qswitch_mid_bytes(T, k, I, E)), dtype=torch.uint8, device=x_expert.device)
    d = gate_up.desc()
    _check(lib().qswitch_gate_up_geglu(_ptr(x_expert), T, H, ctypes.byref(d), I, k, _ptr(expert_offsets),
                                       _ptr(sorted_assign), _ptr(mid), _nbytes(mid), _stream()))
    return mid


def device_status(reset: bool = True) -> int:
    """The device status word (0: no kernel gave up a bounded wait since the
    last reset).  Synchronises the device."""
    v = ctypes.c_int32(0)
    _check(lib().qmoe_device_status(ctypes.byref(v), 1 if reset else 0))
    return int(v.value)


def qswitch_down_combine_workspace(T: int, k: int, H: int, deterministic: int = 1) -> int:
    return int(lib().qswitch_down_combine_workspace(T, k, H, deterministic))


def qswitch_down_combine(mid: torch.Tensor, T: int, k: int, down: "TiledWeight", weights: torch.Tensor,
                         expert_offsets: torch.Tensor, sorted_assign: torch.Tensor,
                         y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         deterministic: int = 1) -> torch.Tensor:
    """down switch linear + weighted sum over k: returns y bf16 [T, H].  mid is the
    activation-tile buffer qswitch_gate_up_geglu wrote."""
    I = down.in_features
    H = down.rows
    E = down.experts
    _need(mid, "mid", 1)
    _need(weights, "weights (fp32)", 4, (T, k))
    _need(expert_offsets, "expert_offsets", 4, (E + 1,))
    _need(sorted_assign, "sorted_assign", 4, (T * k,))
    _need_opt(y, "y", 2, (T, H))
    _need_opt(workspace, "workspace", 1)
    if T > 0 and _nbytes(mid) < qswitch_mid_bytes(T, k, I, E):
        raise ValueError(f"mid: {_nbytes(mid)} bytes, {qswitch_mid_bytes(T, k, I, E)} needed")
    dev = mid.device
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    need = qswitch_down_combine_workspace(T, k, H, deterministic)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = down.desc()
    _check(lib().qswitch_down_combine(_ptr(mid), T, k, I, ctypes.byref(d), H, _ptr(expert_offsets),
                                      _ptr(sorted_assign), _ptr(weights), _ptr(y), _ptr(workspace), ws_bytes,
                                      int(deterministic), _stream()))
    return y


NOALLOC_SCRATCH_BYTES = 16 << 20  # the scratch the library holds per device for the no-allocation calls


def qswitch_down_combine_noalloc(mid: torch.Tensor, T: int, k: int, down: "TiledWeight", weights: torch.Tensor,
                                 expert_offsets: torch.Tensor, sorted_assign: torch.Tensor, y: torch.Tensor,
                                 deterministic: int = 1) -> torch.Tensor:
    """qswitch_down_combine with the library's own scratch instead of a
    workspace: allocates nothing (y is the caller's).  T*k*H*2 bytes of
    scratch at most NOALLOC_SCRATCH_BYTES; calls overlapping on one device
    race."""
    I = down.in_features
    H = down.rows
    E = down.experts
    _need(mid, "mid", 1)
    _need(weights, "weights (fp32)", 4, (T, k))
    _need(expert_offsets, "expert_offsets", 4, (E + 1,))
    _need(sorted_assign, "sorted_assign", 4, (T * k,))
    _need(y, "y", 2, (T, H))
    if T > 0 and _nbytes(mid) < qswitch_mid_bytes(T, k, I, E):
        raise ValueError(f"mid: {_nbytes(mid)} bytes, {qswitch_mid_bytes(T, k, I, E)} needed")
    d = down.desc()
    _check(lib().qswitch_down_combine_noalloc(_ptr(mid), T, k, I, ctypes.byref(d), H, _ptr(expert_offsets),
                                              _ptr(sorted_assign), _ptr(weights), _ptr(y), int(deterministic),
                                              _stream()))
    return y


def qlinear(x: torch.Tensor, W: "TiledWeight", y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense 4-bit linear y = x . dequant(W)^T: returns bf16 [M, N]."""
    M = int(x.shape[0])
    _need(x, "x", 2, (M, W.in_features))
    _need_opt(y, "y", 2, (M, W.rows))
    if y is None:
        y = torch.empty((M, W.rows), dtype=torch.bfloat16, device=x.device)
    d = W.desc()
    _check(lib().qlinear(_ptr(x), M, ctypes.byref(d), _ptr(y), _stream()))
    return y


@dataclass
class MoEParams:
    """Device-resident weights of one MoE layer."""

    norm_scale: torch.Tensor           # bf16 [H]
    router: QuantWeight                # [E, H/8], row-major
    per_expert_scale: torch.Tensor     # bf16 [E]
    gate_up: TiledWeight               # [E, 2I, H], tiled with split = I
    down: TiledWeight                  # [E, H, I], tiled with split = 0
    logit_bias: Optional[torch.Tensor] = None  # fp32 [E]

    @classmethod
    def from_rows(cls, norm_scale, router: QuantWeight, per_expert_scale, gate_up: QuantWeight, down: QuantWeight,
                  logit_bias=None) -> "MoEParams":
        """Tiles the two switch weights (once, when the layer is loaded)."""
        return cls(norm_scale, router, per_expert_scale, gate_up.tiled(gate_up.rows // 2), down.tiled(0), logit_bias)

    @property
    def E(self) -> int:
        return self.router.rows

    @property
    def I(self) -> int:
        return self.gate_up.rows // 2


def moe_layer(x_router: torch.Tensor, x_expert: torch.Tensor, p: MoEParams, k: int, eps: float,
              deterministic: int = 1):
    """The four calls in order.  Returns (y, indices, weights, offsets, sorted_assign, mid)."""
    idx, w = moe_route(x_router, p.norm_scale, eps, p.router, p.per_expert_scale, k, p.logit_bias)
    off, sa = moe_sort(idx, p.E)
    mid = qswitch_gate_up_geglu(x_expert, p.gate_up, p.I, k, off, sa)
    y = qswitch_down_combine(mid, x_expert.shape[0], k, p.down, w, off, sa, deterministic=deterministic)
    return y, idx, w, off, sa, mid


# ----------------------------------------------------------------------------
# the decoder's feed-forward block around the MoE
# ----------------------------------------------------------------------------
def ff_prenorm(h: torch.Tensor, w_dense: torch.Tensor, w_moe: torch.Tensor, eps: float,
               xa: Optional[torch.Tensor] = None, xb: Optional[torch.Tensor] = None):
    """Both pre-norms from one read of h: returns (rms(h) * w_dense, rms(h) * w_moe), bf16 [T, H]."""
    _need(h, "h", 2)
    T, H = (int(v) for v in h.shape)
    _need(w_dense, "w_dense", 2, (H,))
    _need(w_moe, "w_moe", 2, (H,))
    if xa is None:
        xa = torch.empty((T, H), dtype=torch.bfloat16, device=h.device)
    if xb is None:
        xb = torch.empty((T, H), dtype=torch.bfloat16, device=h.device)
    _need(xa, "xa", 2, (T, H))
    _need(xb, "xb", 2, (T, H))
    _check(lib().ff_prenorm(_ptr(h), T, H, _ptr(w_dense), _ptr(w_moe), float(eps), _ptr(xa), _ptr(xb), _stream()))
    return xa, xb


def qlinear_geglu(x: torch.Tensor, W: "TiledWeight", y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gelu_tanh(x . gate^T) * (x . up^T) against the fused [gate; up] weight
    (tiled with split = N): returns bf16 [M, N]."""
    M = int(x.shape[0])
    _need(x, "x", 2, (M, W.in_features))
    _need_opt(y, "y", 2, (M, W.split))
    if y is None:
        y = torch.empty((M, W.split), dtype=torch.bfloat16, device=x.device)
    d = W.desc()
    _check(lib().qlinear_geglu(_ptr(x), M, ctypes.byref(d), _ptr(y), _stream()))
    return y


def ff_combine(h: torch.Tensor, dense_out: torch.Tensor, moe_out: torch.Tensor, w_post1: torch.Tensor,
               w_post2: torch.Tensor, w_post: torch.Tensor, eps: float, layer_scalar: float,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(h + rms(rms(dense_out) w_post1 + rms(moe_out) w_post2) w_post) * layer_scalar, bf16 [T, H]."""
    _need(h, "h", 2)
    T, H = (int(v) for v in h.shape)
    _need(dense_out, "dense_out", 2, (T, H))
    _need(moe_out, "moe_out", 2, (T, H))
    for t, n in ((w_post1, "w_post1"), (w_post2, "w_post2"), (w_post, "w_post")):
        _need(t, n, 2, (H,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=h.device)
    _need(out, "out", 2, (T, H))
    _check(lib().ff_combine(_ptr(h), _ptr(dense_out), _ptr(moe_out), T, H, _ptr(w_post1), _ptr(w_post2),
                            _ptr(w_post), float(eps), float(layer_scalar), _ptr(out), _stream()))
    return out


@dataclass
class FFParams:
    """Device-resident weights of the feed-forward block (besides the MoE's)."""

    pre_ff: torch.Tensor      # bf16 [H]  preFfNorm (dense branch)
    pre_ff2: torch.Tensor     # bf16 [H]  preFfNorm2 (experts)
    post_ff1: torch.Tensor    # bf16 [H]
    post_ff2: torch.Tensor    # bf16 [H]
    post_ff: torch.Tensor     # bf16 [H]
    gate_up: TiledWeight      # [2 I_dense, H]: gate rows then up rows, tiled with split = I_dense
    down: TiledWeight         # [H, I_dense], tiled with split = 0
    layer_scalar: float

    @classmethod
    def from_rows(cls, pre_ff, pre_ff2, post_ff1, post_ff2, post_ff, gate: QuantWeight, up: QuantWeight,
                  down: QuantWeight, layer_scalar: float) -> "FFParams":
        """Stacks gate over up and tiles both linears (once, when the layer is loaded)."""
        if gate.rows != up.rows or gate.in_features != up.in_features:
            raise ValueError("gate and up must have the same shape")
        fused = QuantWeight(torch.cat([gate.w, up.w], dim=-2).contiguous(),
                            torch.cat([gate.scales, up.scales], dim=-2).contiguous(),
                            torch.cat([gate.biases, up.biases], dim=-2).contiguous())
        return cls(pre_ff, pre_ff2, post_ff1, post_ff2, post_ff, fused.tiled(gate.rows), down.tiled(0),
                   float(layer_scalar))


def ff_block(h: torch.Tensor, moe: MoEParams, ff: FFParams, k: int, eps: float, deterministic: int = 1):
    """The feed-forward half of a decoder layer: returns (out bf16 [T, H], indices, weights)."""
    xa, xb = ff_prenorm(h, ff.pre_ff, ff.pre_ff2, eps)
    dense = qlinear(qlinear_geglu(xa, ff.gate_up), ff.down)
    y, idx, w, _, _, _ = moe_layer(h, xb, moe, k, eps, deterministic)
    out = ff_combine(h, dense, y, ff.post_ff1, ff.post_ff2, ff.post_ff, eps, ff.layer_scalar)
    return out, idx, w


# ----------------------------------------------------------------------------
# the unsorted small-batch arm
# ----------------------------------------------------------------------------
def qswitch_unsorted_workspace(T: int, k: int, H: int, I: int) -> int:
    return int(lib().qswitch_unsorted_workspace(T, k, H, I))


def unsorted_workspace(T: int, k: int, H: int, I: int, device="cuda") -> torch.Tensor:
    """Scratch for the unsorted calls (fp32 partial sums; any contents)."""
    n = qswitch_unsorted_workspace(T, k, H, I)
    if n == 0:
        raise ValueError(f"no unsorted workspace for T={T} k={k} H={H} I={I}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def qswitch_gate_up_geglu_unsorted(x_expert: torch.Tensor, gate_up: "TiledWeight", I: int, indices: torch.Tensor,
                                   workspace: torch.Tensor, mid_rows: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gate_up + split + GeGLU per assignment, no sort: returns mid_rows bf16 [T*k, I]."""
    _need(x_expert, "x_expert", 2)
    T, H = (int(v) for v in x_expert.shape)
    k = int(indices.shape[-1])
    _need(indices, "indices", 4, (T, k))
    _same(gate_up.in_features, H, "gate_up in_features vs x_expert.shape[1]")
    _same(gate_up.rows, 2 * I, "gate_up rows vs 2 * I")
    _need(workspace, "workspace", 1)
    if mid_rows is None:
        mid_rows = torch.empty((T * k, I), dtype=torch.bfloat16, device=x_expert.device)
    _need(mid_rows, "mid_rows", 2, (T * k, I))
    d = gate_up.desc()
    _check(lib().qswitch_gate_up_geglu_unsorted(_ptr(x_expert), T, H, ctypes.byref(d), I, k, _ptr(indices),
                                                _ptr(mid_rows), _ptr(workspace), _nbytes(workspace), _stream()))
    return mid_rows


def qswitch_down_combine_unsorted(mid_rows: torch.Tensor, T: int, k: int, down: "TiledWeight", indices: torch.Tensor,
                                  weights: torch.Tensor, workspace: torch.Tensor,
                                  y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """down per assignment + weighted sum over k, no sort: returns y bf16 [T, H]."""
    I = down.in_features
    H = down.rows
    _need(mid_rows, "mid_rows", 2, (T * k, I))
    _need(indices, "indices", 4, (T, k))
    _need(weights, "weights (fp32)", 4, (T, k))
    _need(workspace, "workspace", 1)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=mid_rows.device)
    _need(y, "y", 2, (T, H))
    d = down.desc()
    _check(lib().qswitch_down_combine_unsorted(_ptr(mid_rows), T, k, I, ctypes.byref(d), H, _ptr(indices),
                                               _ptr(weights), _ptr(y), _ptr(workspace), _nbytes(workspace),
                                               _stream()))
    return y


def moe_layer_unsorted(x_router: torch.Tensor, x_expert: torch.Tensor, p: MoEParams, k: int, eps: float,
                       workspace: Optional[torch.Tensor] = None):
    """The small-batch arm: route, then the two unsorted calls.  Returns (y, indices, weights, mid_rows)."""
    T, H = (int(v) for v in x_expert.shape)
    if workspace is None:
        workspace = unsorted_workspace(T, k, H, p.I, device=x_expert.device)
    idx, w = moe_route(x_router, p.norm_scale, eps, p.router, p.per_expert_scale, k, p.logit_bias)
    mid = qswitch_gate_up_geglu_unsorted(x_expert, p.gate_up, p.I, idx, workspace)
    y = qswitch_down_combine_unsorted(mid, T, k, p.down, idx, w, workspace)
    return y, idx, w, mid


# ----------------------------------------------------------------------------
# the tied LM head
# ----------------------------------------------------------------------------
def qlinear_softcap(x: torch.Tensor, W: "TiledWeight", cap: float = 30.0,
                    y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cap * tanh(bf16(x . dequant(W)^T) / cap): returns fp32 [M, N]."""
    M = int(x.shape[0])
    _need(x, "x", 2, (M, W.in_features))
    if y is None:
        y = torch.empty((M, W.rows), dtype=torch.float32, device=x.device)
    _need(y, "y", 4, (M, W.rows))
    d = W.desc()
    _check(lib().qlinear_softcap(_ptr(x), M, ctypes.byref(d), float(cap), _ptr(y), _stream()))
    return y


# ----------------------------------------------------------------------------
# the self-conditioning embedding
# ----------------------------------------------------------------------------
@dataclass
class TiledTWeight:
    """An embedding table [rows, in] re-laid for the untransposed product (qmoe_tile_weight_t)."""

    buf: torch.Tensor
    rows: int
    in_features: int

    def desc(self) -> QWeightDesc:
        _need(self.buf, "tiled table", 1)
        return QWeightDesc(_dptr(self.buf), None, None, 1, self.rows, self.in_features, 4, 64, 2, 0)


def softmax_rows_bf16(z: torch.Tensor, probs: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Precise row softmax of fp32 logits, cast to bf16: returns bf16 [L, V]."""
    _need(z, "z", 4)
    L, V = (int(v) for v in z.shape)
    if probs is None:
        probs = torch.empty((L, V), dtype=torch.bfloat16, device=z.device)
    _need(probs, "probs", 2, (L, V))
    _check(lib().softmax_rows_bf16(_ptr(z), L, V, _ptr(probs), _stream()))
    return probs


def embed_matmul_t(probs: torch.Tensor, W: TiledTWeight, scale: float, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16(bf16(probs . dequant(E)) * scale) with the table E [V, H] used
    without transposing: returns bf16 [L, H]."""
    L = int(probs.shape[0])
    _need(probs, "probs", 2, (L, W.rows))
    _need_opt(workspace, "workspace", 1)
    if out is None:
        out = torch.empty((L, W.in_features), dtype=torch.bfloat16, device=probs.device)
    _need(out, "out", 2, (L, W.in_features))
    if workspace is None:
        workspace = torch.empty(max(1, int(lib().embed_matmul_t_workspace(L, W.rows, W.in_features))),
                                dtype=torch.uint8, device=probs.device)
    d = W.desc()
    _check(lib().embed_matmul_t(_ptr(probs), L, ctypes.byref(d), float(scale), _ptr(out), _ptr(workspace),
                                _nbytes(workspace), _stream()))
    return out


def self_condition_embed(sc_logits: torch.Tensor, W: TiledTWeight, scale: float) -> torch.Tensor:
    """The self-conditioning signal: softmax of the logits to bf16, times the table, times scale."""
    return embed_matmul_t(softmax_rows_bf16(sc_logits), W, scale)

"""Test-side helpers: move seeded numpy inputs to the device and back."""
import os

import numpy as np

import oracle as O


def ensure_built():
    """Build libqmoe.so if it is missing (hipcc cross-compiles without a GPU)."""
    import bit_quantized_moe_diffrouter_amd as q
    if not os.path.exists(q.library_path()):
        from bit_quantized_moe_diffrouter_amd import build
        build.build()
    return q.lib()


def dev_tensor(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def dev_qweight(qt, device="cuda"):
    import bit_quantized_moe_diffrouter_amd as q
    return q.QuantWeight(dev_tensor(qt.w, device), dev_tensor(qt.scales, device), dev_tensor(qt.biases, device))


def dev_params(wt, device="cuda"):
    import bit_quantized_moe_diffrouter_amd as q
    bias = None if wt.logit_bias is None else dev_tensor(wt.logit_bias, device)
    return q.MoEParams.from_rows(dev_tensor(wt.norm_scale, device), dev_qweight(wt.router, device),
                                 dev_tensor(wt.per_expert_scale, device), dev_qweight(wt.gate_up, device),
                                 dev_qweight(wt.down, device), bias)


def bf16_host(t):
    """Device bf16 tensor -> fp64 numpy."""
    import torch
    return O.bf16_to_f64(t.contiguous().view(torch.uint16).cpu().numpy())


def untile_activations(buf, offsets, A, C):
    """Activation-tile buffer (device uint8, layout in qmoe.h) -> fp64 [A, C] in
    sorted-row order, written from the header's description alone: rows of
    expert e's segment in 16-row tiles numbered expert by expert, per (tile,
    64-column group) 2048 bytes where the bf16 at h*1024 + L*16 + 2*i is column
    16*(L//16) + 8*h + i of the group, tile row L % 16.  Rows past offsets[E]
    are zero."""
    import torch
    off = np.asarray(offsets.cpu().numpy() if hasattr(offsets, "cpu") else offsets, dtype=np.int64)
    G = C // 64
    raw = buf.view(torch.uint16).cpu().numpy() if hasattr(buf, "cpu") else np.asarray(buf).view(np.uint16)
    nt_max = raw.size // (G * 1024)
    # [tile, g, h, q, tile row, i] -> [tile, tile row, g, q, h, i] = [tile, 16, C]
    t6 = raw[: nt_max * G * 1024].reshape(nt_max, G, 2, 4, 16, 8)
    tiles = O.bf16_to_f64(t6.transpose(0, 4, 1, 3, 2, 5).reshape(nt_max, 16, C))
    out = np.zeros((A, C))
    tau = 0
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        n = hi - lo
        for j in range((n + 15) // 16):
            r = lo + 16 * j
            m = min(16, hi - r)
            out[r:r + m] = tiles[tau + j, :m]
        tau += (n + 15) // 16
    return out


def say(msg):
    print(msg, flush=True)

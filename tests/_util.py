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


def say(msg):
    print(msg, flush=True)

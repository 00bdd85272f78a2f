"""qswitch_down_combine_noalloc (the library's own scratch, no allocation)
against qswitch_down_combine with a caller workspace, through the C ABI: the
same kernels, so the outputs must agree bit for bit; two calls in a row, the
second on a smaller input, so the second reads what it wrote itself and not
what the first left in the shared scratch."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _util import bf16_host, dev_params, dev_tensor, ensure_built, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    torch.cuda.init()


def prepared(cfg):
    import bit_quantized_moe_diffrouter_amd as q
    inp = synth.make_moe_inputs(cfg)
    p = dev_params(inp.weights)
    x = dev_tensor(inp.x)
    idx, w = q.moe_route(x, p.norm_scale, cfg.eps, p.router, p.per_expert_scale, cfg.k)
    off, sa = q.moe_sort(idx, cfg.E)
    mid = q.qswitch_gate_up_geglu(x, p.gate_up, cfg.I, cfg.k, off, sa)
    return inp, p, idx, w, off, sa, mid


def test_noalloc_matches_workspace_call_twice():
    import bit_quantized_moe_diffrouter_amd as q
    big = synth.CANVAS
    small = synth.MoEConfig("ragged", T=37, H=2816, E=16, k=4, I=704, seed_w=61, seed_x=62)
    assert big.T * big.k * big.H * 2 <= q.NOALLOC_SCRATCH_BYTES
    for cfg in (big, small):
        say(f"[noalloc] {cfg.name}")
        inp, p, idx, w, off, sa, mid = prepared(cfg)
        y_ref = q.qswitch_down_combine(mid, cfg.T, cfg.k, p.down, w, off, sa, deterministic=1)
        y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        q.qswitch_down_combine_noalloc(mid, cfg.T, cfg.k, p.down, w, off, sa, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint16), y_ref.view(torch.uint16))
        toks = list(range(0, cfg.T, max(1, cfg.T // 8)))
        ref = O.experts_bruteforce(inp.x, idx.cpu().numpy(), w.cpu().numpy(), inp.weights.gate_up,
                                   inp.weights.down, cfg.I, tokens=toks)
        assert O.rowwise_rel_err(bf16_host(y)[toks], ref) <= 2e-2


def test_noalloc_rejects_inputs_above_its_scratch():
    import bit_quantized_moe_diffrouter_amd as q
    say("[noalloc] above the limit")
    H, I, E, k = 2816, 704, 128, 8
    T = q.NOALLOC_SCRATCH_BYTES // (k * H * 2) + 1
    inp = synth.make_moe_inputs(synth.MoEConfig("lim", T=1, H=H, E=E, k=k, I=I, seed_w=2, seed_x=3))
    p = dev_params(inp.weights)
    mid = torch.zeros(q.qswitch_mid_bytes(T, k, I, E), dtype=torch.uint8, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    sa = torch.zeros(T * k, dtype=torch.int32, device="cuda")
    y = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QMoEError, match="scratch"):
        q.qswitch_down_combine_noalloc(mid, T, k, p.down, w, off, sa, y)
    torch.cuda.synchronize()
    assert not torch.any(y.float() != 0)

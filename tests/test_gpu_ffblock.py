"""GPU parity of the decoder's feed-forward block around the MoE: the two norm
kernels, the dense GeGLU linear, and the whole block through the bindings,
against the CPU oracle on the same seeded inputs.

Bars (per-row relative error, max |gpu - ref| / max |ref| over a row):
- ff_prenorm, ff_combine: 8e-3.  Each output is one bf16 rounding (2^-9
  relative) of an fp32 result whose own error is far below it; the combine's
  output also carries the bf16 rounding of its inputs' norms through the sum.
- qlinear_geglu: 1e-2, the bar of the experts' GeGLU stage (same kernel
  arithmetic: exact dequant, fp32 accumulate, bf16 store).
- the block: 2e-2, the layer's bound; the GPU rounds to bf16 between its calls
  while the oracle keeps fp64 throughout."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _util import bf16_host, dev_params, dev_qweight, dev_tensor, ensure_built, say

pytestmark = pytest.mark.gpu

NORM_TOL = 8e-3
GEGLU_TOL = 1e-2
BLOCK_TOL = 2e-2
GAP_EXEMPT = 1e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    torch.cuda.init()


_cache = {}


def ff_inputs(cfg):
    """(moe inputs, ff weights) of a feed-forward block config, cached."""
    if cfg.name not in _cache:
        _cache[cfg.name] = (synth.make_moe_inputs(cfg.moe), synth.make_ff_weights(cfg))
    return _cache[cfg.name]


def dev_ff(fw):
    import bit_quantized_moe_diffrouter_amd as q
    d = dev_tensor
    return q.FFParams.from_rows(d(fw.pre_ff), d(fw.pre_ff2), d(fw.post_ff1), d(fw.post_ff2), d(fw.post_ff),
                                dev_qweight(fw.gate), dev_qweight(fw.up), dev_qweight(fw.down), fw.layer_scalar)


def bf16_bits(rng, shape, scale=1.0):
    return synth.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def sample(n_all, n, seed):
    if n_all <= n:
        return list(range(n_all))
    return sorted(np.random.default_rng(seed).choice(n_all, size=n, replace=False).tolist())


# ---------------------------------------------------------------- norms
# rows of up to 4096 columns stay in registers; 4104 and 6144 take the re-reading form
@pytest.mark.parametrize("T,H", [(16, 256), (256, 2816), (37, 72), (1, 8), (5, 2824), (9, 4096), (7, 4104),
                                 (3, 6144)])
def test_ff_prenorm_parity(T, H):
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[ff_prenorm] T={T} H={H}")
    rng = np.random.default_rng(T * 7919 + H)
    h = bf16_bits(rng, (T, H), 3.0)
    wa = synth.to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    wb = synth.to_bf16_bits(rng.uniform(-1.0, 1.0, H).astype(np.float32))
    xa, xb = q.ff_prenorm(dev_tensor(h), dev_tensor(wa), dev_tensor(wb), 1e-6)
    torch.cuda.synchronize()
    for got, w in ((xa, wa), (xb, wb)):
        err = O.rowwise_rel_err(bf16_host(got), O.rms_norm(h, w, 1e-6))
        say(f"  rel err {err:.3e}")
        assert err <= NORM_TOL


@pytest.mark.parametrize("T,H", [(16, 256), (256, 2816), (37, 72), (1, 8), (5, 2824), (9, 4096), (7, 4104),
                                 (3, 6144)])
def test_ff_combine_parity(T, H):
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[ff_combine] T={T} H={H}")
    rng = np.random.default_rng(T * 104729 + H)
    h = bf16_bits(rng, (T, H), 2.0)
    d1 = bf16_bits(rng, (T, H), 0.3)   # branch outputs of different magnitudes
    d2 = bf16_bits(rng, (T, H), 5.0)
    w1, w2, w = (synth.to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32)) for _ in range(3))
    scalar = 0.75
    out = q.ff_combine(dev_tensor(h), dev_tensor(d1), dev_tensor(d2), dev_tensor(w1), dev_tensor(w2),
                       dev_tensor(w), 1e-6, scalar)
    torch.cuda.synchronize()
    s = O.rms_norm(d1, w1, 1e-6) + O.rms_norm(d2, w2, 1e-6)
    ref = (O.bf16_to_f64(h) + O.rms_norm(s, w, 1e-6)) * scalar
    err = O.rowwise_rel_err(bf16_host(out), ref)
    say(f"  rel err {err:.3e}")
    assert err <= NORM_TOL


def test_ff_norms_of_a_zero_branch_row_use_eps():
    """A branch row of zeros normalises to zero (eps > 0): out = (h + N(N1(d1))) * scalar."""
    import bit_quantized_moe_diffrouter_amd as q
    T, H = 4, 256
    rng = np.random.default_rng(3)
    h = bf16_bits(rng, (T, H))
    d1 = bf16_bits(rng, (T, H))
    d2 = np.zeros((T, H), dtype=np.uint16)
    w1, w2, w = (synth.to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32)) for _ in range(3))
    out = q.ff_combine(dev_tensor(h), dev_tensor(d1), dev_tensor(d2), dev_tensor(w1), dev_tensor(w2),
                       dev_tensor(w), 1e-6, 1.0)
    torch.cuda.synchronize()
    ref = O.bf16_to_f64(h) + O.rms_norm(O.rms_norm(d1, w1, 1e-6), w, 1e-6)
    assert np.isfinite(bf16_host(out)).all()
    assert O.rowwise_rel_err(bf16_host(out), ref) <= NORM_TOL


# ---------------------------------------------------------------- dense GeGLU
@pytest.mark.parametrize("M,K,N", [(16, 256, 192), (37, 320, 128), (1, 64, 64), (100, 1152, 448), (65, 128, 576),
                                   (33, 192, 48), (70, 256, 208)])
def test_qlinear_geglu_parity(M, K, N):
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[qlinear_geglu] M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 31 + K * 17 + N)
    gate = synth.random_qtensor(rng, (N,), K)
    up = synth.random_qtensor(rng, (N,), K)
    x = synth.make_activations(M, K, seed=M + K)
    fused = q.QuantWeight(torch.cat([dev_tensor(gate.w), dev_tensor(up.w)]),
                          torch.cat([dev_tensor(gate.scales), dev_tensor(up.scales)]),
                          torch.cat([dev_tensor(gate.biases), dev_tensor(up.biases)])).tiled(N)
    y = q.qlinear_geglu(dev_tensor(x), fused)
    torch.cuda.synchronize()
    err = O.rowwise_rel_err(bf16_host(y), O.dense_geglu(x, gate, up))
    say(f"  rel err {err:.3e}")
    assert err <= GEGLU_TOL


def test_qlinear_geglu_canvas_sampled_rows():
    """The dense branch's first half at the canvas shape (256 x 2816 -> 2112),
    checked on sampled rows."""
    import bit_quantized_moe_diffrouter_amd as q
    cfg = synth.FF_CANVAS
    say(f"[qlinear_geglu] {cfg.name}")
    inp, fw = ff_inputs(cfg)
    ff = dev_ff(fw)
    y = q.qlinear_geglu(dev_tensor(inp.x), ff.gate_up)
    torch.cuda.synchronize()
    rows = sample(cfg.moe.T, 24, seed=11)
    err = O.rowwise_rel_err(bf16_host(y)[rows], O.dense_geglu(inp.x, fw.gate, fw.up, rows=rows))
    say(f"  rel err {err:.3e}")
    assert err <= GEGLU_TOL


# ---------------------------------------------------------------- the block
def run_block(cfg):
    import bit_quantized_moe_diffrouter_amd as q
    inp, fw = ff_inputs(cfg)
    p = dev_params(inp.weights)
    ff = dev_ff(fw)
    out, idx, w = q.ff_block(dev_tensor(inp.x), p, ff, cfg.moe.k, cfg.moe.eps)
    torch.cuda.synchronize()
    return inp, fw, bf16_host(out), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("cfg,n_tok", [(synth.FF_TINY, 16), (synth.FF_CANVAS, 48)], ids=lambda v: getattr(v, "name", v))
def test_ff_block_parity(cfg, n_tok):
    """The whole block through the bindings against the oracle's block; the
    oracle's expert stage takes the GPU's routing (so that near-tied top-k
    choices cannot differ), and the routing itself is checked against the
    oracle's on every token whose k-th/k+1-th logit gap exceeds 1e-5."""
    say(f"[ff_block] {cfg.name}")
    inp, fw, out, idx_g, w_g = run_block(cfg)
    toks = sample(cfg.moe.T, n_tok, seed=13)
    ref, _, _ = O.ff_block(inp.x, inp.weights, fw, cfg.moe.k, cfg.moe.I, cfg.moe.eps, tokens=toks,
                           route_out=(idx_g, w_g))
    err = O.rowwise_rel_err(out[toks], ref)
    say(f"  block rel err {err:.3e} over {len(toks)} tokens")
    assert err <= BLOCK_TOL
    wt, r = inp.weights, inp.weights.router
    idx_r, w_r, lg_r = O.route(inp.x, wt.norm_scale, cfg.moe.eps, r.w, r.scales, r.biases, wt.per_expert_scale,
                               cfg.moe.k, wt.logit_bias)
    ok = O.gap_kth(lg_r, cfg.moe.k) >= GAP_EXEMPT
    assert all(set(idx_g[t]) == set(idx_r[t]) for t in np.nonzero(ok)[0])


def test_ff_block_dense_branch_matches_the_oracle_branch():
    """h1's input on its own: prenorm -> qlinear_geglu -> qlinear at the tiny
    shape, against the oracle's dense branch on the normalised input."""
    import bit_quantized_moe_diffrouter_amd as q
    cfg = synth.FF_TINY
    inp, fw = ff_inputs(cfg)
    ff = dev_ff(fw)
    xa, _ = q.ff_prenorm(dev_tensor(inp.x), ff.pre_ff, ff.pre_ff2, cfg.moe.eps)
    dense = q.qlinear(q.qlinear_geglu(xa, ff.gate_up), ff.down)
    torch.cuda.synchronize()
    ref = O.dense_geglu_mlp(O.rms_norm(inp.x, fw.pre_ff, cfg.moe.eps), fw.gate, fw.up, fw.down)
    err = O.rowwise_rel_err(bf16_host(dense), ref)
    say(f"  dense branch rel err {err:.3e}")
    assert err <= BLOCK_TOL


def test_qlinear_geglu_vision_mlp_width_sampled_rows():
    """The vision tower's MLP gate|up at its geometry: 2520 x 1152 -> 4304, a
    width that is a multiple of 16 but not of 64 (the last tiled block is
    three-quarters empty); sampled rows, every column."""
    import bit_quantized_moe_diffrouter_amd as q
    M, K, N = 2520, 1152, 4304
    say(f"[qlinear_geglu] vision MLP {M}x{K} -> {N}")
    rng = np.random.default_rng(41)
    gate = synth.random_qtensor(rng, (N,), K)
    up = synth.random_qtensor(rng, (N,), K)
    x = synth.make_activations(M, K, seed=42)
    fused = q.QuantWeight(torch.cat([dev_tensor(gate.w), dev_tensor(up.w)]),
                          torch.cat([dev_tensor(gate.scales), dev_tensor(up.scales)]),
                          torch.cat([dev_tensor(gate.biases), dev_tensor(up.biases)])).tiled(N)
    y = q.qlinear_geglu(dev_tensor(x), fused)
    torch.cuda.synchronize()
    rows = [0, 1, 31, 32, 1000, 2495, 2519]
    err = O.rowwise_rel_err(bf16_host(y)[rows], O.dense_geglu(x, gate, up, rows=rows))
    say(f"  rel err {err:.3e}")
    assert err <= GEGLU_TOL

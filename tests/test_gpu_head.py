"""GPU parity of the tied LM head (qlinear_softcap) against the CPU oracle.

Bar: per-row relative error 1e-2 (the GPU rounds an fp32 sum to bf16, the
oracle an fp64 one, so a logit can land one bf16 step apart before the cap).
Special cases: an integer-exact head (every logit a small integer) agrees
with the oracle to fp32 rounding of the tanh; with a huge cap the head is the
bf16 qlinear."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _util import bf16_host, dev_qweight, dev_tensor, ensure_built, say

pytestmark = pytest.mark.gpu

VOCAB = 262144  # the Gemma vocabulary (the pages print an image token id of 258880 but not the size)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    torch.cuda.init()


def head(x_bits, W, cap):
    import bit_quantized_moe_diffrouter_amd as q
    y = q.qlinear_softcap(dev_tensor(x_bits), dev_qweight(W).tiled(0), cap)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,K,N", [(16, 256, 1024), (37, 320, 400), (1, 64, 16), (100, 1152, 2064)])
def test_head_parity(M, K, N):
    say(f"[head] M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 7 + K + N)
    W = synth.random_qtensor(rng, (N,), K)
    x = synth.make_activations(M, K, seed=M + N)
    got = head(x, W, 30.0)
    ref = O.lm_head_softcap(x, W.w, W.scales, W.biases, 30.0)
    err = O.rowwise_rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert err <= 1e-2
    assert np.abs(got).max() < 30.0 + 1e-5


def test_head_canvas_full_vocab_sampled():
    """256 canvas rows against the full 262,144-row head; sampled rows and columns."""
    import bit_quantized_moe_diffrouter_amd as q
    M, K = 256, 2816
    say(f"[head] canvas {M}x{K} -> {VOCAB}")
    rng = np.random.default_rng(12)
    W = synth.random_qtensor(rng, (VOCAB,), K)
    x = synth.make_activations(M, K, seed=13)
    Wt = dev_qweight(W).tiled(0)
    y = q.qlinear_softcap(dev_tensor(x), Wt, 30.0)
    torch.cuda.synchronize()
    rows = [0, 1, 77, 128, 255]
    cols = sorted(np.random.default_rng(14).choice(VOCAB, size=512, replace=False).tolist()) + [VOCAB - 1]
    got = y[rows][:, cols].cpu().numpy().astype(np.float64)
    ref = O.lm_head_softcap(x, W.w[cols], W.scales[cols], W.biases[cols], 30.0, rows=rows)
    err = O.rowwise_rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert err <= 1e-2
    assert bool(torch.isfinite(y).all())


def test_head_integer_exact_logits():
    """Codes, scales, biases and x small integers: every logit is an exact
    small integer, so both sides cap the same z."""
    M, K, N = 8, 128, 64
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(N, K))
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for c in range(8):
        words |= (codes[:, c::8].astype(np.uint32) << (4 * c))
    scales = O.f64_to_bf16_bits(np.ones((N, K // 64)))
    biases = O.f64_to_bf16_bits(np.full((N, K // 64), -8.0))
    W = synth.QTensor(words, scales, biases)
    x = O.f64_to_bf16_bits(rng.integers(-1, 2, size=(M, K)).astype(np.float64))
    z = O.qlinear(x, words, scales, biases)
    assert np.all(np.abs(z) <= 256) and np.array_equal(z, np.round(z))   # exact in bf16
    got = head(x, W, 30.0)
    ref = O.softcap(z, 30.0)
    assert np.abs(got - ref).max() <= 4e-6


def test_head_with_huge_cap_is_the_bf16_qlinear():
    import bit_quantized_moe_diffrouter_amd as q
    M, K, N = 37, 192, 320
    rng = np.random.default_rng(8)
    W = synth.random_qtensor(rng, (N,), K)
    x = synth.make_activations(M, K, seed=9)
    Wt = dev_qweight(W).tiled(0)
    capped = q.qlinear_softcap(dev_tensor(x), Wt, 1e30)
    plain = q.qlinear(dev_tensor(x), Wt)
    torch.cuda.synchronize()
    a = capped.cpu().numpy().astype(np.float64)
    b = bf16_host(plain)
    assert np.allclose(a, b, rtol=1e-6, atol=0)


@pytest.mark.parametrize("M,K", [(100, 128), (17, 192), (64, 64), (129, 128), (300, 192), (520, 64), (256, 576),
                                 (300, 704)])
def test_head_wide_ragged_rows_sampled(M, K):
    """A wide head (131,072 rows of weights, enough items to fill the chip
    without splitting the contraction) at ragged row counts: 100 (three full
    32-row chunks and one of 4 rows), 17 (a second tile holding one row), 64;
    from 128 rows the weight-stationary kernel: 129 (a 128-row tile and one
    row), 300 (a 256-row tile and a ragged one), 520; and at 9 and 11 groups
    (longer than its ring of codes, which every group passes through in
    turn); sampled columns, every row."""
    import bit_quantized_moe_diffrouter_amd as q
    N = 131072
    say(f"[head] wide M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K)
    W = synth.random_qtensor(rng, (N,), K)
    x = synth.make_activations(M, K, seed=M * 3 + 1)
    y = q.qlinear_softcap(dev_tensor(x), dev_qweight(W).tiled(0), 30.0)
    torch.cuda.synchronize()
    cols = sorted(np.random.default_rng(M).choice(N, size=384, replace=False).tolist()) + [N - 1]
    got = y[:, cols].cpu().numpy().astype(np.float64)
    ref = O.lm_head_softcap(x, W.w[cols], W.scales[cols], W.biases[cols], 30.0)
    err = O.rowwise_rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert err <= 1e-2

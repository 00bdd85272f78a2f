"""Hand-worked examples that pin the oracle's router scale, logit offset, the
weighted sum over k and the feed-forward block's norm placement.

Every expected value below is worked out by hand in the docstring next to it
(integer weights, so each logit and each matmul is a short sum), not by
re-running the oracle's formulas.  Each example also runs against a planted
mistake (a wrong input standing in for a wrong oracle step, or a mutated
oracle function patched in for the test) and must then fail: a pin that a
plausible slip would still pass pins nothing.

Passages: [model page] DiffRouter.forward (norm, times the per-dim scale,
times H^-0.5, projection, offset, top-k, precise softmax, per_expert_scale);
DiffExperts.forward (the weighted sum of the k expert outputs per token);
DiffDecoderLayer.forwardWith (preFfNorm before the dense MLP, preFfNorm2
before the experts, the router on the raw residual, postFfNorm1 and
postFfNorm2 on the two branches, postFfNorm on their sum, then the residual
and the layer scalar)."""
import math

import numpy as np
import pytest

import oracle as O
import synth


# ----------------------------------------------------------------------------
# test-side builders (integer weights: scale 1, bias -8, so W = q - 8)
# ----------------------------------------------------------------------------
def bf16(v):
    return synth.to_bf16_bits(np.asarray(v, dtype=np.float32))


def pack(codes):
    codes = np.asarray(codes, dtype=np.uint32)
    out = np.zeros(codes.shape[:-1] + (codes.shape[-1] // 8,), dtype=np.uint32)
    for c in range(codes.shape[-1]):
        out[..., c // 8] |= codes[..., c] << np.uint32(4 * (c % 8))
    return out


def int_weight(W):
    """Integer matrix W (values -8..7, [..., rows, K]) as a 4-bit tensor."""
    W = np.asarray(W)
    G = W.shape[-1] // 64
    lead = W.shape[:-1] + (G,)
    return synth.QTensor(pack(W + 8), bf16(np.ones(lead)), bf16(np.full(lead, -8.0)))


def expect_fail(check, *args, **kw):
    with pytest.raises(AssertionError):
        check(*args, **kw)


# ----------------------------------------------------------------------------
# 1. router: a per-dim scale that is not uniform
# ----------------------------------------------------------------------------
H1 = 64
X_ALT = np.array([1.0 if h % 2 == 0 else -1.0 for h in range(H1)])   # +1 on even h, -1 on odd h
S_PATTERN = np.array([[1.0, 2.0, 0.5, 1.0][h % 4] for h in range(H1)])  # scale by h mod 4


def scale_router():
    """Five experts, integer weights:
    e0: +1 everywhere;       e1: +1 where h % 4 == 1;   e2: -1 where h % 4 == 1;
    e3: +2 where h % 4 == 2; e4: +1 at h = 0 only."""
    W = np.zeros((5, H1), dtype=np.int64)
    W[0] = 1
    W[1, 1::4] = 1
    W[2, 1::4] = -1
    W[3, 2::4] = 2
    W[4, 0] = 1
    return int_weight(W)


def check_router_scale(norm_scale, prologue=None):
    """mean(x^2) = 1, so u_h = x_h s_h / (8 d) with d = sqrt(1 + eps).  Per block
    of four dims x s = (1, -2, 0.5, -1); there are 16 blocks:
      l0 = 16 (1 - 2 + 0.5 - 1) / (8d) = -3/d
      l1 = 16 (-2) / (8d) = -4/d          l2 = +4/d
      l3 = 16 (0.5 * 2) / (8d) = 2/d      l4 = 1 / (8d) = 0.125/d
    top-2 = (e2, e3); p = softmax(4/d, 2/d), p0 = 1 / (1 + exp(-2/d));
    per_expert_scale (1, 1, 0.75, 0.5, 1) gives w = (0.75 p0, 0.5 (1 - p0))."""
    eps = 1e-6
    d = math.sqrt(1 + eps)
    r = scale_router()
    pes = bf16([1.0, 1.0, 0.75, 0.5, 1.0])
    if prologue is not None:
        u = prologue(bf16(X_ALT[None]), norm_scale, eps)
        logits = O.router_logits(u, r.w, r.scales, r.biases)
    else:
        idx, wts, logits = O.route(bf16(X_ALT[None]), norm_scale, eps, r.w, r.scales, r.biases, pes, 2)
        assert idx.tolist() == [[2, 3]]
        p0 = 1.0 / (1.0 + math.exp(-2.0 / d))
        np.testing.assert_allclose(wts[0], [0.75 * p0, 0.5 * (1.0 - p0)], rtol=1e-6)
    np.testing.assert_allclose(logits[0], np.float32([-3 / d, -4 / d, 4 / d, 2 / d, 0.125 / d]), rtol=1e-6)


def test_router_nonuniform_scale_worked_example():
    check_router_scale(bf16(S_PATTERN))
    check_router_scale(bf16(S_PATTERN), prologue=O.router_prologue)


def test_router_scale_example_catches_planted_mistakes():
    # the scale left out (all ones), or divided instead of multiplied
    expect_fail(check_router_scale, bf16(np.ones(H1)))
    expect_fail(check_router_scale, bf16(1.0 / S_PATTERN))

    def scale_before_norm(x_bits, s_bits, eps):  # the scale applied before the norm
        x = O.bf16_to_f64(x_bits) * O.bf16_to_f64(s_bits)
        return O.rms_norm_noscale(x, eps) * float(np.float32(x.shape[-1] ** -0.5))

    expect_fail(check_router_scale, bf16(S_PATTERN), prologue=scale_before_norm)


# ----------------------------------------------------------------------------
# 2. router: a per-expert logit offset that changes the set and the weights
# ----------------------------------------------------------------------------
def offset_router():
    """e0: W = x (+1 on even h, -1 on odd h);  e1: 0;  e2: W = -x;  e3: +1 at h = 0."""
    W = np.zeros((4, H1), dtype=np.int64)
    W[0] = X_ALT.astype(np.int64)
    W[2] = -X_ALT.astype(np.int64)
    W[3, 0] = 1
    return int_weight(W)


OFFSET = np.float32([0.0, 9.0, 0.0, 0.5])


def check_router_offset(route_fn=None):
    """Scale 1, mean(x^2) = 1, u = x / (8d):  l = (8/d, 0, -8/d, 0.125/d), plus
    the offset (0, 9, 0, 0.5) -> (8/d, 9, -8/d, 0.125/d + 0.5).  top-2 = (e1, e0)
    (without the offset it would be e0, e3); p1 = 1 / (1 + exp(8/d - 9));
    per_expert_scale (1, 0.5, 1, 1) gives w = (0.5 p1, 1 - p1)."""
    eps = 1e-6
    d = math.sqrt(1 + eps)
    r = offset_router()
    pes = bf16([1.0, 0.5, 1.0, 1.0])
    fn = route_fn or O.route
    idx, wts, logits = fn(bf16(X_ALT[None]), bf16(np.ones(H1)), eps, r.w, r.scales, r.biases, pes, 2, OFFSET)
    np.testing.assert_allclose(logits[0], np.float32([8 / d, 9.0, -8 / d, 0.125 / d + 0.5]), rtol=1e-6)
    assert idx.tolist() == [[1, 0]]
    p1 = 1.0 / (1.0 + math.exp(8.0 / d - 9.0))
    np.testing.assert_allclose(wts[0], [0.5 * p1, 1.0 - p1], rtol=1e-6)


def test_router_logit_offset_worked_example():
    check_router_offset()


def test_router_offset_example_catches_planted_mistakes():
    def offset_after_topk(x, s, eps, w, sc, b, pes, k, bias):  # selection on the raw logits
        u = O.router_prologue(x, s, eps)
        raw = O.router_logits(u, w, sc, b)
        idx = O.top_k(raw, k)
        biased = raw.astype(np.float64) + bias
        p = O.precise_softmax(np.take_along_axis(biased, idx, axis=-1))
        return idx, (p * O.bf16_to_f64(pes)[idx]).astype(np.float32), biased.astype(np.float32)

    def offset_not_in_softmax(x, s, eps, w, sc, b, pes, k, bias):  # softmax over the raw logits
        u = O.router_prologue(x, s, eps)
        raw = O.router_logits(u, w, sc, b)
        biased = O.router_logits(u, w, sc, b, bias)
        idx = O.top_k(biased, k)
        p = O.precise_softmax(np.take_along_axis(raw.astype(np.float64), idx, axis=-1))
        return idx, (p * O.bf16_to_f64(pes)[idx]).astype(np.float32), biased

    expect_fail(check_router_offset, offset_after_topk)
    expect_fail(check_router_offset, offset_not_in_softmax)
    expect_fail(check_router_offset, lambda *a: O.route(*a[:-1], None))  # the offset left out


# ----------------------------------------------------------------------------
# 3. experts: E = 2, k = 2, the weighted sum over the k slots
# ----------------------------------------------------------------------------
def two_experts():
    """H = I = 64, x = 4 e_0 for both tokens.  Expert e: gate row 0 is +7 at
    h = 0, so gate_0 = 28 and gelu_tanh(28) = 28 exactly (its tanh is 1.0 in
    double); up row 0 is +1 (e0) or +3 (e1) at h = 0, so up_0 = 4 or 12 and
    mid = (112, 0, ...) for e0, (336, 0, ...) for e1; every other row is 0.
    Down: e0 has +1 at (0, 0) and -1 at (1, 0), so d0 = (112, -112, 0, ...);
    e1 has +2 at (1, 0), so d1 = (0, 672, 0, ...)."""
    H, I = 64, 64
    gu = np.zeros((2, 2 * I, H), dtype=np.int64)
    dn = np.zeros((2, H, I), dtype=np.int64)
    gu[:, 0, 0] = 7
    gu[0, I, 0] = 1
    gu[1, I, 0] = 3
    dn[0, 0, 0] = 1
    dn[0, 1, 0] = -1
    dn[1, 1, 0] = 2
    x = np.zeros((2, H))
    x[:, 0] = 4.0
    return bf16(x), int_weight(gu), int_weight(dn), I


IDX2 = np.array([[0, 1], [1, 0]], dtype=np.int32)
W2 = np.float32([[0.5, 0.25], [0.5, 0.25]])


def check_two_expert_sum(weights, fn):
    """token 0: 0.5 d0 + 0.25 d1 = (56, -56 + 168) = (56, 112);
    token 1: 0.5 d1 + 0.25 d0 = (28, 336 - 28) = (28, 308); the rest 0."""
    x, gu, dn, I = two_experts()
    y = np.asarray(fn(x, IDX2, weights, gu, dn, I), dtype=np.float64)
    expect = np.zeros((2, 64))
    expect[0, :2] = (56.0, 112.0)
    expect[1, :2] = (28.0, 308.0)
    np.testing.assert_array_equal(y, expect)


@pytest.mark.parametrize("fn", [O.experts_bruteforce, O.experts_grouped], ids=["bruteforce", "grouped"])
def test_two_experts_weighted_sum_worked_example(fn):
    check_two_expert_sum(W2, fn)


@pytest.mark.parametrize("fn", [O.experts_bruteforce, O.experts_grouped], ids=["bruteforce", "grouped"])
def test_two_expert_example_catches_planted_mistakes(fn):
    expect_fail(check_two_expert_sum, W2 / 2, fn)           # the mean over k instead of the sum
    expect_fail(check_two_expert_sum, W2[:, ::-1].copy(), fn)  # weight j paired with slot 1 - j


def test_two_expert_mid_and_down_pieces():
    """mid of assignments (t, j): e0 rows give 112 in column 0, e1 rows 336."""
    x, gu, dn, I = two_experts()
    mid = O.expert_mid_bruteforce(x, IDX2, gu, I, [0, 1, 2, 3])
    assert mid[:, 0].tolist() == [112.0, 336.0, 336.0, 112.0]
    assert not np.any(mid[:, 1:])
    y = O.down_combine_from_mid(mid, IDX2, W2, dn, [0, 1])
    assert y[:, :2].tolist() == [[56.0, 112.0], [28.0, 308.0]]


# ----------------------------------------------------------------------------
# 4. the feed-forward block: which norm weight goes where, router on raw h
# ----------------------------------------------------------------------------
def ff_example():
    """H = 64, one token h = 1 everywhere, eps = 0 (so every norm below is exact).

    Norm weights: preFfNorm a = (1 x 32, 2 x 32); postFfNorm1 = 3;
    preFfNorm2 b = (4 x 32, 1 x 32); postFfNorm2 = 5; postFfNorm = 6;
    layer scalar 0.5.

    Router (k = 1, scale 1): e0 +1 everywhere, e1 +2 on the first half and
    -1 on the second.  On the raw h, u = 1/8 per dim: l = (8, 4), so e0 with
    weight per_expert_scale[0] = 1.  (On preFfNorm2(h) = b it would be e1.)

    Expert e0 on b: gate rows 0, 1 are +7 everywhere: 7 * 160 = 1120 (its
    gelu_tanh is exactly 1120); up row 0 is +1 on dims 0..31 -> 128, up row 1
    is +1 on dims 0..15 and 32..47 -> 80; down maps mid 0 -> dim 2 and mid
    1 -> dim 3: m2 = 1120 (0, 0, 128, 80, 0, ...), rms(m2) = 1120 sqrt(356),
    h2 = 5 m2 / rms = (0, 0, 640, 400) / sqrt(356).  (Expert e1 writes dim 4.)

    Dense branch on a: gate rows 0, 1 are +7 everywhere: 7 * 96 = 672; up
    row 0 is +1 on dims 0..31 -> 32, up row 1 +1 on dims 32..63 -> 64; down
    maps mid j -> dim j: m1 = 672 (32, 64, 0, ...), rms(m1) = 21504 sqrt(5) / 8,
    h1 = 3 m1 / rms = (24, 48) / sqrt(5).

    s = h1 + h2 has mean(s^2) = (2880/5 + 569600/356) / 64 = 34, so
    out = 0.5 (1 + 6 s / sqrt(34)):
      out_0 = 0.5 + 72/sqrt(170),    out_1 = 0.5 + 144/sqrt(170),
      out_2 = 0.5 + 1920/sqrt(12104), out_3 = 0.5 + 1200/sqrt(12104), else 0.5."""
    H, I, Id = 64, 64, 64
    half = np.arange(H) < 32
    a = np.where(half, 1.0, 2.0)
    b = np.where(half, 4.0, 1.0)
    ffw_norms = dict(pre_ff=bf16(a), post_ff1=bf16(np.full(H, 3.0)), pre_ff2=bf16(b),
                     post_ff2=bf16(np.full(H, 5.0)), post_ff=bf16(np.full(H, 6.0)))
    Wr = np.zeros((2, H), dtype=np.int64)
    Wr[0] = 1
    Wr[1] = np.where(half, 2, -1)
    gu = np.zeros((2, 2 * I, H), dtype=np.int64)
    dn = np.zeros((2, H, I), dtype=np.int64)
    gu[0, 0] = 7
    gu[0, 1] = 7
    gu[0, I] = half.astype(np.int64)
    gu[0, I + 1] = ((np.arange(H) % 32) < 16).astype(np.int64)
    dn[0, 2, 0] = 1
    dn[0, 3, 1] = 1
    gu[1, 0] = 7
    gu[1, I] = 1
    dn[1, 4, 0] = 1
    moe = synth.MoEWeights(bf16(np.ones(H)), int_weight(Wr), bf16([1.0, 0.5]), int_weight(gu), int_weight(dn))
    g = np.zeros((Id, H), dtype=np.int64)
    u = np.zeros((Id, H), dtype=np.int64)
    d = np.zeros((H, Id), dtype=np.int64)
    g[0] = 7
    g[1] = 7
    u[0] = half.astype(np.int64)
    u[1] = (~half).astype(np.int64)
    d[0, 0] = 1
    d[1, 1] = 1
    ffw = synth.FFWeights(gate=int_weight(g), up=int_weight(u), down=int_weight(d), layer_scalar=0.5, **ffw_norms)
    return bf16(np.ones((1, H))), moe, ffw, I


def ff_expected():
    out = np.full(64, 0.5)
    out[0] = 0.5 + 72 / math.sqrt(170)
    out[1] = 0.5 + 144 / math.sqrt(170)
    out[2] = 0.5 + 1920 / math.sqrt(12104)
    out[3] = 0.5 + 1200 / math.sqrt(12104)
    return out


def check_ff(h, moe, ffw, I, route_out=None):
    out, idx, wts = O.ff_block(h, moe, ffw, 1, I, 0.0, route_out=route_out)
    if route_out is None:
        assert idx.tolist() == [[0]] and wts.tolist() == [[1.0]]
    np.testing.assert_allclose(out[0], ff_expected(), rtol=1e-12, atol=1e-12)


def test_ff_block_norm_placement_worked_example():
    check_ff(*ff_example())


def test_ff_block_example_catches_planted_mistakes():
    import dataclasses
    h, moe, ffw, I = ff_example()
    swap = dataclasses.replace
    expect_fail(check_ff, h, moe, swap(ffw, pre_ff=ffw.pre_ff2, pre_ff2=ffw.pre_ff), I)
    expect_fail(check_ff, h, moe, swap(ffw, post_ff1=ffw.post_ff2, post_ff2=ffw.post_ff1), I)
    # the router fed preFfNorm2(h) instead of the raw residual
    hn = bf16(O.rms_norm(h, ffw.pre_ff2, 0.0))
    r = moe.router
    idx, wts, _ = O.route(hn, moe.norm_scale, 0.0, r.w, r.scales, r.biases, moe.per_expert_scale, 1)
    assert idx.tolist() == [[1]]
    expect_fail(check_ff, h, moe, ffw, I, route_out=(idx, wts))
    # norms with a 1 + w offset
    plus1 = lambda v: bf16(O.bf16_to_f64(v) + 1.0)
    expect_fail(check_ff, h, moe, swap(ffw, post_ff=plus1(ffw.post_ff)), I)

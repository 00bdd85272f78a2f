"""Pins for the CPU oracle: every check compares it with something other than
itself -- hand-worked golden files, closed forms, integer arithmetic, brute
force on tiny inputs, textbook special cases and invariants of the method."""
import math
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# test-side helpers, written independently of the oracle
# ----------------------------------------------------------------------------
def pack_codes_loop(codes):
    """Pack codes [rows, K] (ints 0..15) into uint32 words, first code lowest."""
    rows, K = codes.shape
    out = np.zeros((rows, K // 8), dtype=np.uint32)
    for r in range(rows):
        for c in range(K):
            out[r, c // 8] |= np.uint32(int(codes[r, c]) << (4 * (c % 8)))
    return out


def bf16(v):
    return synth.to_bf16_bits(np.asarray(v, dtype=np.float32))


def integer_qtensor(codes):
    """Weights with scale 1 and bias -8, so W = q - 8 exactly."""
    rows, K = codes.shape
    G = K // 64
    return (pack_codes_loop(codes), bf16(np.ones((rows, G))), bf16(np.full((rows, G), -8.0)))


# ----------------------------------------------------------------------------
# Q: packing and dequantization
# ----------------------------------------------------------------------------
def test_nibble_order_golden():
    with open(os.path.join(GOLDEN, "nibble_order.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    words = np.array([int(r[0], 16) for r in rows], dtype=np.uint32)
    expect = np.array([[int(v) for v in r[1:]] for r in rows], dtype=np.uint8)
    got = O.unpack_codes(words.reshape(-1, 1))
    np.testing.assert_array_equal(got, expect)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=(5, 128))
    np.testing.assert_array_equal(O.unpack_codes(pack_codes_loop(codes)), codes)


def test_dequant_group_structure():
    # all codes 1, bias 0, scale of group g = g + 1  ->  W[c] = c // 64 + 1
    K = 256
    codes = np.ones((3, K), dtype=np.int64)
    w = pack_codes_loop(codes)
    s = bf16(np.tile(np.arange(1, K // 64 + 1), (3, 1)))
    b = bf16(np.zeros((3, K // 64)))
    W = O.dequantize(w, s, b)
    expect = np.tile(np.arange(K) // 64 + 1, (3, 1)).astype(np.float64)
    np.testing.assert_array_equal(W, expect)


def test_dequant_invariant_scale_q_bias():
    """Spec invariant: the unpacked weight equals scale*q + bias per
    64-wide group.  Checked element by element with codes from the test-side
    packer (not the oracle's unpacker)."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, size=(4, 192))
    w = pack_codes_loop(codes)
    sf = rng.uniform(0.01, 0.05, size=(4, 3)).astype(np.float32)
    bf_ = rng.uniform(-0.4, 0.1, size=(4, 3)).astype(np.float32)
    s, b = bf16(sf), bf16(bf_)
    sd, bd = synth.bf16_bits_as_f32(s).astype(np.float64), synth.bf16_bits_as_f32(b).astype(np.float64)
    W = O.dequantize(w, s, b)
    for n in range(4):
        for c in range(0, 192, 7):
            assert W[n, c] == sd[n, c // 64] * codes[n, c] + bd[n, c // 64]


def test_all_eights_with_minus_eight_scale_bias_is_zero():
    K = 128
    codes = np.full((6, K), 8)
    w = pack_codes_loop(codes)
    s = bf16(np.abs(np.random.default_rng(3).normal(0, 0.02, size=(6, 2))))
    b = bf16(-8.0 * synth.bf16_bits_as_f32(s))
    assert not np.any(O.dequantize(w, s, b))
    x = bf16(np.random.default_rng(4).standard_normal((3, K)))
    assert not np.any(O.qlinear(x, w, s, b))


def test_qlinear_integer_exact():
    """scale 1, bias -8, x in {-2..2}: y is an integer matmul (exact)."""
    rng = np.random.default_rng(13)
    M, N, K = 9, 40, 192
    codes = rng.integers(0, 16, size=(N, K))
    xi = rng.integers(-2, 3, size=(M, K))
    w, s, b = integer_qtensor(codes)
    y = O.qlinear(bf16(xi), w, s, b)
    expect = xi.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    np.testing.assert_array_equal(y, expect.astype(np.float64))


# ----------------------------------------------------------------------------
# R: router
# ----------------------------------------------------------------------------
def test_rms_norm_constant_row_closed_form():
    for c in (0.5, -3.0, 1e-3):
        x = np.full((1, 128), c)
        r = O.rms_norm_noscale(x, 1e-6)
        np.testing.assert_allclose(r, c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_router_worked_example_closed_form():
    """H = 64, E = 4, k = 2, x alternating +1/-1, norm scale 1, integer router
    weights.  mean(x^2) = 1, so u = x / sqrt(1 + eps) / 8 and the logits are
    l_e = sum_h x_h (q_eh - 8) / (8 sqrt(1 + eps)):
    e0: q = 9 on +1, 7 on -1 -> 64/8;  e1: q = 8 -> 0;
    e2: q = 7 on +1, 9 on -1 -> -64/8;  e3: q = 9 at h = 0 only -> 1/8."""
    H, eps = 64, 1e-6
    x = np.array([1.0 if h % 2 == 0 else -1.0 for h in range(H)])
    q = np.full((4, H), 8)
    q[0] = np.where(x > 0, 9, 7)
    q[2] = np.where(x > 0, 7, 9)
    q[3, 0] = 9
    w, s, b = integer_qtensor(q)
    pes = bf16([1.0, 1.0, 1.0, 0.5])
    idx, wts, logits = O.route(bf16(x[None]), bf16(np.ones(H)), eps, w, s, b, pes, 2)
    d = math.sqrt(1 + eps)
    np.testing.assert_allclose(logits[0], np.float32([8 / d, 0.0, -8 / d, 0.125 / d]), rtol=1e-7)
    assert idx.tolist() == [[0, 3]]
    p0 = 1.0 / (1.0 + math.exp(-(8 - 0.125) / d))
    np.testing.assert_allclose(wts[0], [p0, 0.5 * (1 - p0)], rtol=1e-6)


def topk_selection_loop(row, k):
    vals = list(map(float, row))
    taken, out = set(), []
    for _ in range(k):
        best = None
        for e, v in enumerate(vals):
            if e in taken:
                continue
            if best is None or v > vals[best]:
                best = e
        taken.add(best)
        out.append(best)
    return out


def test_topk_matches_selection_loop_with_ties():
    rng = np.random.default_rng(14)
    logits = rng.integers(-3, 4, size=(40, 12)).astype(np.float32) * 0.25  # many ties
    for k in (1, 3, 8, 12):
        got = O.top_k(logits, k)
        for t in range(logits.shape[0]):
            assert got[t].tolist() == topk_selection_loop(logits[t], k)


def test_topk_special_cases():
    rng = np.random.default_rng(15)
    logits = rng.standard_normal((20, 16)).astype(np.float32)
    np.testing.assert_array_equal(O.top_k(logits, 1)[:, 0], np.argmax(logits, axis=1))
    full = O.top_k(logits, 16)
    for t in range(20):
        assert sorted(full[t].tolist()) == list(range(16))
        assert np.all(np.diff(logits[t, full[t]]) <= 0)


def test_softmax_invariants():
    rng = np.random.default_rng(16)
    v = rng.standard_normal((50, 8)) * 3
    p = O.precise_softmax(v)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    np.testing.assert_allclose(O.precise_softmax(v + 7.25), p, atol=1e-15)
    np.testing.assert_allclose(O.precise_softmax(np.zeros((3, 8))), 1.0 / 8)
    assert np.all(p > 0)


def test_route_weights_sum_to_one_before_per_expert_scale():
    cfg = synth.TINY
    inp = synth.make_moe_inputs(cfg)
    r = inp.weights.router
    ones = bf16(np.ones(cfg.E))
    _, w1, _ = O.route(inp.x, inp.weights.norm_scale, cfg.eps, r.w, r.scales, r.biases, ones, cfg.k)
    np.testing.assert_allclose(w1.astype(np.float64).sum(-1), 1.0, atol=1e-6)
    idx, w, _ = O.route(inp.x, inp.weights.norm_scale, cfg.eps, r.w, r.scales, r.biases,
                        inp.weights.per_expert_scale, cfg.k)
    pes = synth.bf16_bits_as_f32(inp.weights.per_expert_scale)
    np.testing.assert_allclose(w, w1 * pes[idx], rtol=1e-6)
    assert np.all(w >= 0) and np.all(w <= pes.max())


# ----------------------------------------------------------------------------
# S: sort
# ----------------------------------------------------------------------------
def read_kv(path):
    out = {}
    with open(path) as f:
        for l in f:
            if l.strip() and not l.startswith("#"):
                key, *vals = l.split()
                out[key] = [int(v) for v in vals]
    return out


def test_sort_golden():
    g = read_kv(os.path.join(GOLDEN, "sort_small.txt"))
    idx = np.array(g["indices"], dtype=np.int32).reshape(-1, g["k"][0])
    off, sa = O.sort_assignments(idx, g["E"][0])
    assert off.tolist() == g["offsets"]
    assert sa.tolist() == g["sorted_assign"]


def counting_sort_loop(flat, E):
    buckets = [[] for _ in range(E)]
    for a, e in enumerate(flat):
        buckets[e].append(a)
    offs = [0]
    for b in buckets:
        offs.append(offs[-1] + len(b))
    return offs, [a for b in buckets for a in b]


def test_sort_matches_counting_sort_loop():
    rng = np.random.default_rng(17)
    for T, k, E in [(16, 2, 8), (33, 4, 10), (64, 8, 128), (1, 1, 1)]:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        off, sa = O.sort_assignments(idx, E)
        offs, order = counting_sort_loop(idx.reshape(-1).tolist(), E)
        assert off.tolist() == offs
        assert sa.tolist() == order
        inv = np.empty_like(sa)
        inv[sa] = np.arange(sa.size)
        np.testing.assert_array_equal(sa[inv], np.arange(sa.size))


# ----------------------------------------------------------------------------
# X: GELU and the expert path
# ----------------------------------------------------------------------------
def test_gelu_tanh_pins():
    from scipy.special import erf
    assert O.gelu_tanh(0.0) == 0.0
    z = np.linspace(-8, 8, 4001)
    g = O.gelu_tanh(z)
    np.testing.assert_allclose(g - O.gelu_tanh(-z), z, atol=1e-12)  # odd-part identity
    exact = 0.5 * z * (1 + erf(z / math.sqrt(2)))
    assert np.abs(g - exact).max() < 5e-4  # the tanh form's known error (about 4.7e-4)
    np.testing.assert_allclose(O.gelu_tanh(np.array([30.0, -30.0])), [30.0, 0.0], atol=1e-12)


def test_grouped_equals_bruteforce_on_tiny():
    cfg = synth.TINY
    inp = synth.make_moe_inputs(cfg)
    wt = inp.weights
    y, idx, w, _ = O.moe_layer(inp.x, wt, cfg.k, cfg.I, cfg.eps, grouped=True)
    yb = O.experts_bruteforce(inp.x, idx, w, wt.gate_up, wt.down, cfg.I)
    assert O.rowwise_rel_err(y, yb) < 1e-5
    assert y.shape == (cfg.T, cfg.H)


def test_single_expert_reduces_to_dense_geglu_mlp():
    """E = 1, k = 1: y = per_expert_scale[0] * down(gelu(gate(x)) * up(x)),
    computed here with integer weights and plain numpy."""
    rng = np.random.default_rng(18)
    T, H, I = 5, 128, 64
    cg = rng.integers(0, 16, size=(2 * I, H))
    cd = rng.integers(0, 16, size=(H, I))
    gu = synth.QTensor(*[a[None] for a in integer_qtensor(cg)])
    dn = synth.QTensor(*[a[None] for a in integer_qtensor(cd)])
    xf = rng.integers(-2, 3, size=(T, H)).astype(np.float64) * 0.125
    x = bf16(xf)
    idx = np.zeros((T, 1), dtype=np.int32)
    pes = 1.25
    w = np.full((T, 1), pes, dtype=np.float32)
    y = O.experts_bruteforce(x, idx, w, gu, dn, I)
    Wg = cg.astype(np.float64) - 8
    Wd = cd.astype(np.float64) - 8
    g = xf @ Wg.T
    a = g[:, :I]
    mid = 0.5 * a * (1 + np.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3))) * g[:, I:]
    np.testing.assert_allclose(y, pes * (mid @ Wd.T), rtol=1e-12, atol=1e-9)


def test_layer_token_equivariance_and_duplicates():
    cfg = synth.TINY
    inp = synth.make_moe_inputs(cfg)
    wt = inp.weights
    y, *_ = O.moe_layer(inp.x, wt, cfg.k, cfg.I, cfg.eps, grouped=False)
    perm = np.random.default_rng(19).permutation(cfg.T)
    yp, *_ = O.moe_layer(inp.x[perm], wt, cfg.k, cfg.I, cfg.eps, grouped=False)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-12, atol=1e-12)
    xd = np.concatenate([inp.x[:3], inp.x[:3]])
    yd, *_ = O.moe_layer(xd, wt, cfg.k, cfg.I, cfg.eps, grouped=False)
    np.testing.assert_array_equal(yd[:3], yd[3:])


def test_layer_linear_in_down_projection():
    cfg = synth.TINY
    inp = synth.make_moe_inputs(cfg)
    wt = inp.weights
    y, idx, w, _ = O.moe_layer(inp.x, wt, cfg.k, cfg.I, cfg.eps, grouped=False)
    d = wt.down
    d2 = synth.QTensor(d.w, bf16(2.0 * synth.bf16_bits_as_f32(d.scales)),
                       bf16(2.0 * synth.bf16_bits_as_f32(d.biases)))
    y2 = O.experts_bruteforce(inp.x, idx, w, wt.gate_up, d2, cfg.I)
    np.testing.assert_array_equal(y2, 2.0 * y)


def test_mid_and_down_pieces_compose_to_layer():
    cfg = synth.TINY
    inp = synth.make_moe_inputs(cfg)
    wt = inp.weights
    y, idx, w, _ = O.moe_layer(inp.x, wt, cfg.k, cfg.I, cfg.eps, grouped=False)
    A = cfg.T * cfg.k
    mid = O.expert_mid_bruteforce(inp.x, idx, wt.gate_up, cfg.I, list(range(A)))
    y2 = O.down_combine_from_mid(mid, idx, w, wt.down, list(range(cfg.T)))
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)


def test_rowwise_rel_err_metric():
    ref = np.array([[1.0, -2.0], [0.5, 0.25]])
    y = ref + np.array([[0.02, 0.0], [0.0, 0.01]])
    assert abs(O.rowwise_rel_err(y, ref) - 0.02) < 1e-15


def test_bf16_roundtrip_and_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.140625], dtype=np.float64)
    bits = O.f64_to_bf16_bits(v)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    np.testing.assert_array_equal(O.bf16_to_f64(bits), [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 3.140625])


# ----------------------------------------------------------------------------
# F: the decoder's feed-forward block
# ----------------------------------------------------------------------------
def test_rms_norm_weighted_closed_form():
    """A constant row c*1 normalises to c / sqrt(c^2 + eps) before the weight;
    the stored weight multiplies as is (a 1 + w offset would double these)."""
    eps = 1e-6
    w = np.array([0.5, 1.0, 1.5, 2.0] * 16, dtype=np.float32)
    for c in (3.0, -0.25, 1e-4):
        x = np.full((1, 64), c)
        y = O.rms_norm(x, bf16(w), eps)
        np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * w.astype(np.float64), rtol=1e-12)
    # a worked row: x = (3, 4, 0, 0), mean(x^2) = 25/4, so r = x / 2.5 (eps 0)
    y = O.rms_norm(np.array([[3.0, 4.0, 0.0, 0.0]]), bf16([1.0, 2.0, 1.0, 1.0]), 0.0)
    np.testing.assert_allclose(y, [[1.2, 3.2, 0.0, 0.0]], rtol=1e-12)


def test_rms_norm_scale_invariant_and_zero_row():
    rng = np.random.default_rng(40)
    x = rng.standard_normal((3, 128))
    w = bf16(rng.uniform(0.8, 1.2, 128))
    # exact invariance with eps = 0 (eps shifts it by about eps / mean(x^2))
    np.testing.assert_allclose(O.rms_norm(37.0 * x, w, 0.0), O.rms_norm(x, w, 0.0), rtol=1e-12)
    assert np.all(O.rms_norm(np.zeros((1, 128)), w, 1e-6) == 0.0)


def test_dense_geglu_mlp_integer_worked_example():
    """Integer weights (W = q - 8) and x in eighths: gate, up and down by plain
    numpy; swapping gate and up, or transposing a weight, changes the result."""
    rng = np.random.default_rng(41)
    H, Id = 128, 64
    cg, cu = rng.integers(0, 16, size=(Id, H)), rng.integers(0, 16, size=(Id, H))
    cd = rng.integers(0, 16, size=(H, Id))
    gate = synth.QTensor(*integer_qtensor(cg))
    up = synth.QTensor(*integer_qtensor(cu))
    down = synth.QTensor(*integer_qtensor(cd))
    xf = rng.integers(-2, 3, size=(4, H)).astype(np.float64) * 0.125
    y = O.dense_geglu_mlp(bf16(xf), gate, up, down)
    g = xf @ (cg - 8.0).T
    u = xf @ (cu - 8.0).T
    ref = (0.5 * g * (1 + np.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3))) * u) @ (cd - 8.0).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-9)
    swapped = O.dense_geglu_mlp(bf16(xf), up, gate, down)
    assert np.abs(swapped - ref).max() > 1.0


def test_ff_block_with_zero_branches_is_scaled_residual():
    """All codes 8 with bias -8*scale make every 4-bit weight zero: both
    branches vanish, their norms map 0 to 0, and out = h * layer_scalar."""
    cfg = synth.FF_TINY
    inp = synth.make_moe_inputs(cfg.moe)
    ffw = synth.make_ff_weights(cfg)
    eights = lambda qt: synth.QTensor(np.full_like(qt.w, 0x88888888), qt.scales, qt.biases)
    wt = inp.weights
    zero_moe = synth.MoEWeights(wt.norm_scale, wt.router, wt.per_expert_scale, eights(wt.gate_up),
                                eights(wt.down), wt.logit_bias)
    zero_ff = synth.FFWeights(ffw.pre_ff, ffw.pre_ff2, ffw.post_ff1, ffw.post_ff2, ffw.post_ff,
                              eights(ffw.gate), eights(ffw.up), eights(ffw.down), ffw.layer_scalar)
    out, _, _ = O.ff_block(inp.x, zero_moe, zero_ff, cfg.moe.k, cfg.moe.I, cfg.moe.eps)
    np.testing.assert_array_equal(out, O.bf16_to_f64(inp.x) * ffw.layer_scalar)


def test_ff_block_residual_raw_branches_scale_invariant():
    """Scaling h by a > 0 leaves the routing (its own norm) and both branches
    (they see normalised copies) unchanged, while the residual enters raw:
    out(a h) - a s h == out(h) - s h."""
    cfg = synth.FF_TINY
    inp = synth.make_moe_inputs(cfg.moe)
    ffw = synth.make_ff_weights(cfg)
    s = ffw.layer_scalar
    h = O.bf16_to_f64(inp.x)
    h4 = bf16(4.0 * h)  # exact: a power of two
    out1, idx1, _ = O.ff_block(inp.x, inp.weights, ffw, cfg.moe.k, cfg.moe.I, cfg.moe.eps)
    out4, idx4, _ = O.ff_block(h4, inp.weights, ffw, cfg.moe.k, cfg.moe.I, cfg.moe.eps)
    np.testing.assert_array_equal(idx1, idx4)
    np.testing.assert_allclose(out4 - 4.0 * s * h, out1 - s * h, rtol=1e-6, atol=1e-6)


def test_ff_block_rows_and_given_routing():
    """Selected rows equal the full block's rows; feeding back the block's own
    routing reproduces it."""
    cfg = synth.FF_TINY
    inp = synth.make_moe_inputs(cfg.moe)
    ffw = synth.make_ff_weights(cfg)
    full, idx, w = O.ff_block(inp.x, inp.weights, ffw, cfg.moe.k, cfg.moe.I, cfg.moe.eps)
    rows = [3, 11, 0]
    part, _, _ = O.ff_block(inp.x, inp.weights, ffw, cfg.moe.k, cfg.moe.I, cfg.moe.eps, tokens=rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-12, atol=1e-12)
    again, _, _ = O.ff_block(inp.x, inp.weights, ffw, cfg.moe.k, cfg.moe.I, cfg.moe.eps, route_out=(idx, w))
    np.testing.assert_allclose(again, full, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------- H: tied head + softcap
def test_softcap_closed_forms():
    cap = 30.0
    z = np.array([-1e6, -45.0, -1.0, 0.0, 0.3, 1.0, 45.0, 1e6])
    y = O.softcap(z, cap)
    assert np.all(np.abs(y) < cap + 1e-12)
    assert np.allclose(O.softcap(-z, cap), -y, rtol=0, atol=0)          # odd
    assert y[0] == -cap and y[-1] == cap                                 # saturates at +-cap
    # tanh(atanh(1/2)) = 1/2: the point where the cap halves
    assert abs(O.softcap(cap * math.atanh(0.5), cap) - cap / 2) < 1e-12
    # small z: z - z^3 / (3 cap^2) + 2 z^5 / (15 cap^4)
    s = 0.01 * cap
    assert abs(O.softcap(s, cap) - (s - s ** 3 / (3 * cap ** 2) + 2 * s ** 5 / (15 * cap ** 4))) < 1e-12


def test_lm_head_with_huge_cap_is_the_bf16_qlinear():
    rng = np.random.default_rng(21)
    W = synth.random_qtensor(rng, (48,), 128)
    x = synth.make_activations(5, 128, seed=3)
    ref = O.bf16_to_f64(O.f64_to_bf16_bits(O.qlinear(x, W.w, W.scales, W.biases)))
    got = O.lm_head_softcap(x, W.w, W.scales, W.biases, cap=1e12)
    assert np.allclose(got, ref, rtol=1e-15, atol=0)
    rows = [4, 0, 2]
    assert np.array_equal(O.lm_head_softcap(x, W.w, W.scales, W.biases, 30.0, rows=rows),
                          O.lm_head_softcap(x, W.w, W.scales, W.biases, 30.0)[rows])


def test_lm_head_rounds_to_bf16_before_the_cap():
    """A logit of 257 (not a bf16 value) is returned as 256 by the quantized
    matmul and only then capped: 30 tanh(256 / 30), not 30 tanh(257 / 30)."""
    # one row of 64 codes 1, scale 1, bias 0 -> weight row of ones; x: 64 values summing to 257
    words = np.full((1, 8), 0x11111111, dtype=np.uint32)
    scales = O.f64_to_bf16_bits(np.ones((1, 1)))
    biases = O.f64_to_bf16_bits(np.zeros((1, 1)))
    xv = np.full((1, 64), 4.0)
    xv[0, 0] = 5.0                                        # 63 * 4 + 5 = 257
    x = O.f64_to_bf16_bits(xv)
    got = O.lm_head_softcap(x, words, scales, biases, 30.0)
    assert abs(got[0, 0] - 30.0 * math.tanh(256.0 / 30.0)) < 1e-12
    assert abs(got[0, 0] - 30.0 * math.tanh(257.0 / 30.0)) > 1e-8


# ---------------------------------------------------------------------------- C: self-conditioning embedding
def test_embed_matmul_t_one_hot_probabilities_pick_a_row():
    """Logits with one value far above the rest give a probability of exactly
    1 there and 0 elsewhere, so the product is that row of the dequantized
    table, rounded to bf16, times the scale, rounded again."""
    rng = np.random.default_rng(31)
    V, H, L = 96, 128, 3
    W = synth.random_qtensor(rng, (V,), H)
    logits = rng.standard_normal((L, V))
    hot = [5, 0, 95]
    for l, v in enumerate(hot):
        logits[l, v] += 2000.0
    p = O.softmax_rows_bf16(logits)
    assert np.array_equal(O.bf16_to_f64(p).sum(axis=1), np.ones(L))
    scale = math.sqrt(2816.0)
    got = O.embed_matmul_t(p, W.w, W.scales, W.biases, scale)
    Wd = O.dequantize(W.w, W.scales, W.biases)
    for l, v in enumerate(hot):
        row = O.bf16_to_f64(O.f64_to_bf16_bits(Wd[v]))
        want = O.bf16_to_f64(O.f64_to_bf16_bits(row * np.float32(scale)))
        assert np.array_equal(got[l], want)


def test_embed_matmul_t_uniform_probabilities_give_column_means():
    """Equal logits over V = 2^k entries give probabilities of exactly 2^-k,
    so the product is the table's column sums times 2^-k."""
    rng = np.random.default_rng(32)
    V, H = 256, 64
    W = synth.random_qtensor(rng, (V,), H)
    p = O.softmax_rows_bf16(np.zeros((2, V)))
    assert np.all(O.bf16_to_f64(p) == 2.0 ** -8)
    got = O.embed_matmul_t(p, W.w, W.scales, W.biases, 1.0)
    cols = O.dequantize(W.w, W.scales, W.biases).sum(axis=0) * 2.0 ** -8
    want = O.bf16_to_f64(O.f64_to_bf16_bits(cols))
    assert np.array_equal(got[0], want) and np.array_equal(got[1], want)
    assert np.array_equal(O.embed_matmul_t(p, W.w, W.scales, W.biases, 1.0, rows=[1]), got[[1]])


# ---------------------------------------------------------------------------- inputs
def test_synth_independent_biases():
    """The general affine workload: biases not a fixed multiple of the scales,
    codes and scales identical to the default stream's."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, bias_seed=101)
    wt, w0 = synth.make_moe_weights(cfg), synth.make_moe_weights(synth.TINY)
    np.testing.assert_array_equal(wt.gate_up.w, w0.gate_up.w)
    np.testing.assert_array_equal(wt.gate_up.scales, w0.gate_up.scales)
    s = synth.bf16_bits_as_f32(wt.gate_up.scales).astype(np.float64)
    b = synth.bf16_bits_as_f32(wt.gate_up.biases).astype(np.float64)
    ratio = b[s > 0] / s[s > 0]
    assert np.std(ratio) > 1.0 and np.mean(b == -8 * s) < 0.05


def test_token_of_multiply_high_is_exact():
    """The switch kernels find the token of assignment a (a // k) as the high
    32 bits of a * (floor(2^32 / k) + 1), for every a below 2^24 (the
    library's limit on T * k) and every k from 2 to 16 (k = 1 is passed
    through).  Checked here on all of them."""
    import numpy as np
    a = np.arange(1 << 24, dtype=np.uint64)
    for k in range(2, 17):
        inv = np.uint64((1 << 32) // k + 1)
        assert np.array_equal((a * inv) >> np.uint64(32), a // np.uint64(k)), k

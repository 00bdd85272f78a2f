"""GPU parity: every call of the C ABI against the CPU oracle on the same
seeded inputs, stage by stage (route, sort, mid, y) and end to end.

Bars: routing indices bit-exact except tokens whose 8th/9th oracle-logit gap
is below 1e-5 (compared as per-token sets, since equal-valued slots may come
out in either order); weights within 1e-5; sort bit-exact; float outputs
within a per-row relative error of 2e-2 (the layer's bound), with tighter
stage bars where the only difference is the bf16 store."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _util import bf16_host, dev_params, dev_qweight, dev_tensor, ensure_built, say, untile_activations

pytestmark = pytest.mark.gpu

GAP_EXEMPT = 1e-5
Y_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    torch.cuda.init()


_cache = {}


def canvas_weights():
    if "w" not in _cache:
        _cache["w"] = synth.make_moe_weights(synth.CANVAS)
    return _cache["w"]


def inputs(cfg):
    if cfg.name in _cache:
        return _cache[cfg.name]
    if cfg.H == 2816:
        w = canvas_weights()
        if cfg.zipf_tau is not None:
            w = synth.MoEWeights(w.norm_scale, w.router, w.per_expert_scale, w.gate_up, w.down,
                                 synth.zipf_logit_bias(cfg.E, cfg.zipf_tau, cfg.zipf_perm_seed))
        inp = synth.make_moe_inputs(cfg, w)
    else:
        inp = synth.make_moe_inputs(cfg)
    _cache[cfg.name] = inp
    return inp


def params(cfg):
    key = ("dev", cfg.name)
    if key not in _cache:
        _cache[key] = dev_params(inputs(cfg).weights)
    return _cache[key]


def oracle_route(inp):
    cfg, wt = inp.cfg, inp.weights
    r = wt.router
    return O.route(inp.x, wt.norm_scale, cfg.eps, r.w, r.scales, r.biases, wt.per_expert_scale, cfg.k,
                   wt.logit_bias)


def gpu_route(inp, p, logits=True):
    import bit_quantized_moe_diffrouter_amd as q
    cfg = inp.cfg
    x = dev_tensor(inp.x)
    lo = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda") if logits else None
    idx, w = q.moe_route(x, p.norm_scale, cfg.eps, p.router, p.per_expert_scale, cfg.k, p.logit_bias,
                         logits_out=lo)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), (lo.cpu().numpy() if logits else None)


def assert_route_parity(inp, idx_g, w_g, lg_g):
    """Logits within 2e-6; outside the exempt band the oracle's set and
    weights; on every token (exempt ones included) a valid top-k of the GPU's
    own logits -- k distinct experts in descending order whose smallest logit
    is at least the largest unselected one -- with weights equal to the
    precise softmax of those selected logits times per_expert_scale."""
    cfg = inp.cfg
    idx_r, w_r, lg_r = oracle_route(inp)
    np.testing.assert_allclose(lg_g, lg_r, rtol=0, atol=2e-6)
    gap = O.gap_kth(lg_r, cfg.k)
    exempt = gap < GAP_EXEMPT
    for t in np.nonzero(~exempt)[0]:
        assert set(idx_g[t].tolist()) == set(idx_r[t].tolist()), f"token {t}: {idx_g[t]} vs {idx_r[t]}"
        wg = dict(zip(idx_g[t].tolist(), w_g[t].tolist()))
        for e, wr in zip(idx_r[t].tolist(), w_r[t].tolist()):
            assert abs(wg[e] - wr) <= 1e-5, f"token {t} expert {e}: {wg[e]} vs {wr}"
    pes = O.bf16_to_f64(inp.weights.per_expert_scale)
    for t in range(cfg.T):
        sel = idx_g[t].tolist()
        assert len(set(sel)) == cfg.k and all(0 <= e < cfg.E for e in sel)
        picked = lg_g[t, sel].astype(np.float64)
        assert np.all(np.diff(picked) <= 0)
        rest = np.delete(lg_g[t], sel)
        if rest.size:
            assert picked.min() >= rest.max(), f"token {t}: selected {picked.min()} < unselected {rest.max()}"
        ref_w = O.precise_softmax(picked) * pes[sel]
        np.testing.assert_allclose(w_g[t], ref_w, rtol=0, atol=1e-6, err_msg=f"token {t}")
    return int(exempt.sum())


MOE_CFGS = [synth.TINY, synth.CANVAS, synth.PREFILL, synth.SKEW]


@pytest.mark.parametrize("cfg", MOE_CFGS, ids=lambda c: c.name)
def test_route_parity(cfg):
    say(f"[route] {cfg.name}")
    inp = inputs(cfg)
    idx_g, w_g, lg_g = gpu_route(inp, params(cfg))
    n_ex = assert_route_parity(inp, idx_g, w_g, lg_g)
    say(f"  exempt tokens: {n_ex}")


def test_route_weights_sum_to_one_before_per_expert_scale():
    cfg = synth.CANVAS
    say(f"[route pes=1] {cfg.name}")
    inp = inputs(cfg)
    p = params(cfg)
    import bit_quantized_moe_diffrouter_amd as q
    ones = dev_tensor(synth.to_bf16_bits(np.ones(cfg.E, dtype=np.float32)))
    _, w = q.moe_route(dev_tensor(inp.x), p.norm_scale, cfg.eps, p.router, ones, cfg.k)
    s = w.double().sum(-1).cpu().numpy()
    assert np.abs(s - 1.0).max() <= 1e-6


@pytest.mark.parametrize("T,H,E,k", [(37, 320, 40, 5), (5, 128, 16, 16), (33, 256, 200, 1), (3, 64, 1, 1),
                                     (21, 192, 256, 16), (1100, 320, 40, 5), (1030, 192, 256, 16),
                                     (1024, 64, 1, 1)])
def test_route_ragged_and_degenerate(T, H, E, k):
    """Ragged token counts (down to a last 16-token tile of 4 or 6 tokens, also
    past 1024 tokens, where the contraction is split in at most 4 parts), expert
    counts that are not multiples of 16, single groups and single experts."""
    say(f"[route ragged] T={T} H={H} E={E} k={k}")
    cfg = synth.MoEConfig("ragged", T=T, H=H, E=E, k=k, I=64, seed_w=7, seed_x=8)
    inp = synth.make_moe_inputs(cfg)
    idx_g, w_g, lg_g = gpu_route(inp, dev_params(inp.weights))
    assert_route_parity(inp, idx_g, w_g, lg_g)
    if k == 1:
        np.testing.assert_array_equal(idx_g[:, 0], np.argmax(lg_g, axis=1))


@pytest.mark.parametrize("E,k,NI_case", [(40, 5, "one key per lane"), (128, 8, "two"), (256, 16, "four")])
def test_route_ties_go_to_the_lower_expert(E, k, NI_case):
    """Router rows repeated (expert e uses row e % 7), so every token's logits
    come in groups of equal values, bitwise equal on the GPU too: the
    selection must be the oracle's tie rule applied to the GPU's own logits
    (descending, equal logits to the lower expert), exactly, with weights the
    softmax of the selected logits times per_expert_scale."""
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[route ties] E={E} k={k} ({NI_case})")
    T, H = 37, 128
    cfg = synth.MoEConfig("ties", T=T, H=H, E=E, k=k, I=64, seed_w=51, seed_x=52)
    inp = synth.make_moe_inputs(cfg)
    r = inp.weights.router
    rep = np.arange(E) % 7
    router = synth.QTensor(r.w[rep], r.scales[rep], r.biases[rep])
    wt = synth.MoEWeights(inp.weights.norm_scale, router, inp.weights.per_expert_scale, inp.weights.gate_up,
                          inp.weights.down)
    p = dev_params(wt)
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx, w = q.moe_route(dev_tensor(inp.x), p.norm_scale, cfg.eps, p.router, p.per_expert_scale, k, logits_out=lo)
    torch.cuda.synchronize()
    lg, idx_g, w_g = lo.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    for t in range(T):
        assert len(set(lg[t].tolist())) <= 7
    np.testing.assert_array_equal(idx_g, O.top_k(lg, k))
    pes = O.bf16_to_f64(wt.per_expert_scale)
    for t in range(T):
        ref = O.precise_softmax(lg[t, idx_g[t]].astype(np.float64)) * pes[idx_g[t]]
        np.testing.assert_allclose(w_g[t], ref, rtol=0, atol=1e-6)


# ------------------------------------------------------------------------- sort
def gpu_sort(idx, E, slices=True):
    import bit_quantized_moe_diffrouter_amd as q
    off, sa = q.moe_sort(dev_tensor(idx.astype(np.int32)), E, slices=slices)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sa.cpu().numpy()


@pytest.mark.parametrize("cfg", MOE_CFGS, ids=lambda c: c.name)
def test_sort_parity(cfg):
    say(f"[sort] {cfg.name}")
    idx_r, _, _ = oracle_route(inputs(cfg))
    off_g, sa_g = gpu_sort(idx_r, cfg.E)
    off_r, sa_r = O.sort_assignments(idx_r, cfg.E)
    np.testing.assert_array_equal(off_g, off_r)
    np.testing.assert_array_equal(sa_g, sa_r)


@pytest.mark.parametrize("slices", [True, False], ids=["slices", "one_workgroup"])
def test_sort_large_random_and_dropped(slices):
    say(f"[sort] random 3000x8 over 256 experts, with out-of-range indices (slices={slices})")
    rng = np.random.default_rng(21)
    T, k, E = 3000, 8, 256
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    off_g, sa_g = gpu_sort(idx, E, slices)
    off_r, sa_r = O.sort_assignments(idx, E)
    np.testing.assert_array_equal(off_g, off_r)
    np.testing.assert_array_equal(sa_g, sa_r)
    bad = idx.copy()
    bad[5, 3] = -1
    bad[17, 0] = E
    bad[2999, 7] = 1 << 20
    off_g, sa_g = gpu_sort(bad, E, slices)
    flat = bad.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    ids = np.nonzero(valid)[0]
    nv = ids.size
    expect_order = ids[np.argsort(flat[ids], kind="stable")]
    expect_off = np.concatenate([[0], np.cumsum(np.bincount(flat[ids], minlength=E))])
    np.testing.assert_array_equal(off_g, expect_off)
    np.testing.assert_array_equal(sa_g[:nv], expect_order)
    np.testing.assert_array_equal(sa_g[nv:], np.nonzero(~valid)[0])



def check_sort(idx, E, off_g, sa_g):
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    ids = np.nonzero(valid)[0]
    np.testing.assert_array_equal(off_g, np.concatenate([[0], np.cumsum(np.bincount(flat[ids], minlength=E))]))
    np.testing.assert_array_equal(sa_g[:ids.size], ids[np.argsort(flat[ids], kind="stable")])
    np.testing.assert_array_equal(sa_g[ids.size:], np.nonzero(~valid)[0])


@pytest.mark.parametrize("slices", [True, False], ids=["slices", "one_workgroup"])
@pytest.mark.parametrize("T,k,E", [(4100, 8, 128), (9000, 4, 7), (18750, 16, 256)])
def test_sort_beyond_the_lds_cache(T, k, E, slices):
    """More than 32768 assignments.  One workgroup recomputes buckets and
    ranks instead of keeping them in LDS; the slice sort cuts the input into
    33, 36 and 147 slices (of 1024, 1024 and 2048 assignments).  Stable order
    and offsets as before."""
    say(f"[sort] beyond the LDS cache: T={T} k={k} E={E} slices={slices}")
    rng = np.random.default_rng(T)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.01] = -3
    off_g, sa_g = gpu_sort(idx, E, slices)
    check_sort(idx, E, off_g, sa_g)


@pytest.mark.parametrize("T,k,E,hot", [(1024, 8, 128, 1.0), (1025, 8, 128, 0.9), (2000, 8, 1, 0.0)])
def test_sort_slices_threshold_and_hot_expert(T, k, E, hot):
    """At and just past the slice sort's threshold (8192 assignments: 8 and 9
    slices, the last one 8 assignments long), with one expert taking all or
    90 % of the assignments (every slice's histogram lands in one LDS bucket),
    and with a single expert; the two sorts give the same bits."""
    say(f"[sort] threshold T={T} k={k} E={E} hot={hot}")
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < hot] = E // 2
    idx[0, 0] = -1
    off_s, sa_s = gpu_sort(idx, E, True)
    off_1, sa_1 = gpu_sort(idx, E, False)
    np.testing.assert_array_equal(off_s, off_1)
    np.testing.assert_array_equal(sa_s, sa_1)
    check_sort(idx, E, off_s, sa_s)


def test_sort_slices_beyond_the_lds_cache():
    """9,000,000 assignments: 252 slices of 35,840, each past its LDS cache,
    so each slice recomputes buckets and ranks in its scatter pass."""
    T, k, E = 562500, 16, 256
    say(f"[sort] slices beyond the LDS cache: T={T} k={k} E={E}")
    rng = np.random.default_rng(99)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.001] = E + 1
    off_g, sa_g = gpu_sort(idx, E, True)
    check_sort(idx, E, off_g, sa_g)


# ------------------------------------------------------------------ experts
def sample_tokens(T, n, seed=5):
    if T <= n:
        return list(range(T))
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(T, size=n, replace=False).tolist())


def run_experts(inp, idx, w, deterministic=1):
    import bit_quantized_moe_diffrouter_amd as q
    cfg = inp.cfg
    p = params(cfg)
    x = dev_tensor(inp.x)
    idx_d = dev_tensor(idx.astype(np.int32))
    w_d = dev_tensor(w.astype(np.float32))
    off, sa = q.moe_sort(idx_d, cfg.E)
    mid = q.qswitch_gate_up_geglu(x, p.gate_up, cfg.I, cfg.k, off, sa)
    y = q.qswitch_down_combine(mid, cfg.T, cfg.k, p.down, w_d, off, sa, deterministic=deterministic)
    torch.cuda.synchronize()
    return bf16_host(y), untile_activations(mid, off, cfg.T * cfg.k, cfg.I), sa.cpu().numpy()


@pytest.mark.parametrize("cfg", MOE_CFGS, ids=lambda c: c.name)
def test_gate_up_mid_parity(cfg):
    say(f"[gate_up mid] {cfg.name}")
    inp = inputs(cfg)
    idx_r, w_r, _ = oracle_route(inp)
    _, mid_g, sa = run_experts(inp, idx_r, w_r)
    A = cfg.T * cfg.k
    rows = list(range(A)) if A <= 64 else sample_tokens(A, 48, seed=9)
    ref = O.expert_mid_bruteforce(inp.x, idx_r, inp.weights.gate_up, cfg.I, [int(sa[r]) for r in rows])
    err = O.rowwise_rel_err(mid_g[rows], ref)
    say(f"  mid rel err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("cfg", MOE_CFGS, ids=lambda c: c.name)
def test_down_combine_parity_from_gpu_mid(cfg):
    """Down + combine checked on its own: the oracle starts from the GPU's
    bf16 mid, so only the down projection and the sum over k are compared."""
    say(f"[down+combine] {cfg.name}")
    inp = inputs(cfg)
    idx_r, w_r, _ = oracle_route(inp)
    y_g, mid_g, sa = run_experts(inp, idx_r, w_r)
    mid_by_assign = np.zeros_like(mid_g)
    mid_by_assign[sa] = mid_g
    toks = sample_tokens(cfg.T, 24)
    ref = O.down_combine_from_mid(mid_by_assign, idx_r, w_r, inp.weights.down, toks)
    err = O.rowwise_rel_err(y_g[toks], ref)
    say(f"  y rel err {err:.3e}")
    assert err <= 1e-2


def mixed_routing(inp, idx_g, w_g):
    """The oracle's own routing, except on tokens inside the exempt band
    (8th/9th oracle-logit gap below 1e-5), which keep the GPU's."""
    idx_r, w_r, lg_r = oracle_route(inp)
    ex = O.gap_kth(lg_r, inp.cfg.k) < GAP_EXEMPT
    idx_m, w_m = idx_r.copy(), w_r.copy()
    idx_m[ex], w_m[ex] = idx_g[ex], w_g[ex]
    return idx_m, w_m, idx_r, ex


@pytest.mark.parametrize("cfg", MOE_CFGS, ids=lambda c: c.name)
def test_layer_parity(cfg):
    """Whole layer through the four calls against the oracle's whole layer:
    the oracle routes every token itself, except those inside the exempt band,
    which take the GPU's routing (there either choice is correct)."""
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[layer] {cfg.name}")
    inp = inputs(cfg)
    p = params(cfg)
    x = dev_tensor(inp.x)
    y, idx, w, off, sa, mid = q.moe_layer(x, x, p, cfg.k, cfg.eps)
    torch.cuda.synchronize()
    idx_g, w_g = idx.cpu().numpy(), w.cpu().numpy()
    idx_m, w_m, idx_r, ex = mixed_routing(inp, idx_g, w_g)
    assert all(set(idx_g[t]) == set(idx_r[t]) for t in np.nonzero(~ex)[0])
    toks = sample_tokens(cfg.T, 32)
    ref = O.experts_bruteforce(inp.x, idx_m, w_m, inp.weights.gate_up, inp.weights.down, cfg.I, tokens=toks)
    err = O.rowwise_rel_err(bf16_host(y)[toks], ref)
    say(f"  layer rel err {err:.3e} over {len(toks)} tokens ({int(ex.sum())} exempt in all)")
    assert err <= Y_TOL


@pytest.mark.parametrize("cfg", [synth.CANVAS, synth.PREFILL, synth.SKEW], ids=lambda c: c.name)
def test_layer_all_tokens_against_grouped_oracle(cfg):
    """Every token of the canvas, the 4096-token prefill and the skewed canvas
    against the fp32 grouped oracle (oracle routing outside the exempt band)."""
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[layer all tokens] {cfg.name}")
    inp = inputs(cfg)
    p = params(cfg)
    x = dev_tensor(inp.x)
    y, idx, w, *_ = q.moe_layer(x, x, p, cfg.k, cfg.eps)
    torch.cuda.synchronize()
    idx_m, w_m, _, ex = mixed_routing(inp, idx.cpu().numpy(), w.cpu().numpy())
    ref = O.experts_grouped(inp.x, idx_m, w_m, inp.weights.gate_up, inp.weights.down, cfg.I)
    err = O.rowwise_rel_err(bf16_host(y), ref)
    say(f"  rel err {err:.3e} over {cfg.T} tokens")
    assert err <= Y_TOL


def test_sorted_layer_in_hip_graph():
    """The sorted layer (route, sort, gate_up, down + combine) on the canvas
    workload captured in a HIP graph, twice over with two token sets: every
    replay, with eager work and synchronisations in between, gives the eager
    result bit for bit (the calls enqueue only kernels)."""
    import bit_quantized_moe_diffrouter_amd as q
    cfg = synth.CANVAS
    say(f"[graph] {cfg.name}")
    inp = inputs(cfg)
    p = params(cfg)
    T, k, H, I, E = cfg.T, cfg.k, cfg.H, cfg.I, cfg.E
    xs = [dev_tensor(inp.x), dev_tensor(synth.make_activations(T, H, 78))]
    dev = "cuda"
    ws_r = torch.empty(q.moe_route_workspace(T, H, E), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(q.qswitch_down_combine_workspace(T, k, H, 1), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(T * k, dtype=torch.int32, device=dev)
    mid = torch.empty(q.qswitch_mid_bytes(T, k, I, E), dtype=torch.uint8, device=dev)
    ys = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in xs]

    def layers():
        for x, y in zip(xs, ys):
            q.moe_route(x, p.norm_scale, cfg.eps, p.router, p.per_expert_scale, k, None, indices=idx, weights=wts,
                        workspace=ws_r)
            q.moe_sort(idx, E, off, sa, workspace=None)
            q.qswitch_gate_up_geglu(x, p.gate_up, I, k, off, sa, mid=mid)
            q.qswitch_down_combine(mid, T, k, p.down, wts, off, sa, y=y, workspace=ws_d, deterministic=1)

    layers()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layers()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layers()
    for rep in range(3):
        for y in ys:
            y.fill_(0)
        q.moe_sort(idx, E)          # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.uint16), e.view(torch.uint16)), f"replay {rep} differs from eager"


def test_layer_deterministic_bitwise():
    import bit_quantized_moe_diffrouter_amd as q
    cfg = synth.CANVAS
    say(f"[determinism] {cfg.name}")
    inp = inputs(cfg)
    p = params(cfg)
    x = dev_tensor(inp.x)
    y1 = q.moe_layer(x, x, p, cfg.k, cfg.eps)[0].clone()
    y2 = q.moe_layer(x, x, p, cfg.k, cfg.eps)[0].clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.uint16), y2.view(torch.uint16))


# (45, 576, 12, 4, 320): gate_up's contraction of 9 groups is split 4 + 5 over a
# wave pair, and the down output ends in a half block (576 = 4.5 x 128);
# (200, 512, 6, 4, 128): experts of ~130 rows, several chunks each, many items
# per worker.
# From 96 rows per expert on average gate_up runs on the tall-tile kernel: (200, 512, 6, 4, 128) and the three below (128-row tiles with a
# ragged last one, empty experts, a single expert with 1000 rows, and a gate
# width of 320 = 5 blocks of 64 columns).
@pytest.mark.parametrize("T,H,E,k,I", [(1, 64, 1, 1, 64), (37, 192, 12, 3, 192), (9, 256, 8, 8, 64),
                                       (45, 576, 12, 4, 320), (200, 512, 6, 4, 128),
                                       (40, 128, 256, 16, 64),  # the largest E and k: 257 buckets in down
                                       (300, 256, 5, 2, 320), (1000, 128, 1, 1, 64), (250, 192, 16, 8, 192)])
def test_layer_ragged_and_degenerate(T, H, E, k, I):
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[layer ragged] T={T} H={H} E={E} k={k} I={I}")
    cfg = synth.MoEConfig("ragged", T=T, H=H, E=E, k=k, I=I, seed_w=31, seed_x=32)
    inp = synth.make_moe_inputs(cfg)
    p = dev_params(inp.weights)
    x = dev_tensor(inp.x)
    y, idx, w, *_ = q.moe_layer(x, x, p, k, cfg.eps)
    torch.cuda.synchronize()
    ref = O.experts_bruteforce(inp.x, idx.cpu().numpy(), w.cpu().numpy(), inp.weights.gate_up,
                               inp.weights.down, I)
    err = O.rowwise_rel_err(bf16_host(y), ref)
    say(f"  rel err {err:.3e}")
    assert err <= Y_TOL


def test_layer_dropped_indices_sum_the_rest():
    """Out-of-range routing indices are dropped: the token gets the weighted
    sum of its remaining assignments."""
    import bit_quantized_moe_diffrouter_amd as q
    cfg = synth.TINY
    say("[layer dropped indices]")
    inp = inputs(cfg)
    idx_r, w_r, _ = oracle_route(inp)
    bad = idx_r.copy()
    bad[3, 1] = -7
    bad[10, 0] = cfg.E
    y_g, _, _ = run_experts(inp, bad, w_r)
    w0 = w_r.copy()
    w0[3, 1] = 0.0
    w0[10, 0] = 0.0
    safe = np.where((bad >= 0) & (bad < cfg.E), bad, 0)
    ref = O.experts_bruteforce(inp.x, safe, w0, inp.weights.gate_up, inp.weights.down, cfg.I)
    assert O.rowwise_rel_err(y_g, ref) <= Y_TOL


def test_zero_tokens_is_a_noop():
    import bit_quantized_moe_diffrouter_amd as q
    say("[T=0]")
    p = params(synth.TINY)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    idx, w = q.moe_route(x, p.norm_scale, 1e-6, p.router, p.per_expert_scale, 2)
    assert idx.shape == (0, 2)


# --------------------------------------------------------------------- qlinear
def test_qlinear_vision_geometry():
    import bit_quantized_moe_diffrouter_amd as q
    cfg = synth.QLINEAR_VISION
    say(f"[qlinear] {cfg.name}")
    inp = synth.make_qlinear_inputs(cfg)
    y = q.qlinear(dev_tensor(inp.x), dev_qweight(inp.W).tiled())
    torch.cuda.synchronize()
    ref = O.qlinear(inp.x, inp.W.w, inp.W.scales, inp.W.biases)
    err = O.rowwise_rel_err(bf16_host(y), ref)
    say(f"  rel err {err:.3e}")
    assert err <= 1e-2


def test_qlinear_integer_exact_bitwise():
    """scale 1, bias -8, x in {-2..2}: the exact integer result rounded once to
    bf16 must come out bit for bit."""
    import bit_quantized_moe_diffrouter_amd as q
    say("[qlinear integer-exact] 2520x1152 -> 1152")
    rng = np.random.default_rng(41)
    M, N, K = 2520, 1152, 1152
    w = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32)
    s = synth.to_bf16_bits(np.ones((N, K // 64), dtype=np.float32))
    b = synth.to_bf16_bits(np.full((N, K // 64), -8.0, dtype=np.float32))
    x = synth.to_bf16_bits(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
    y = q.qlinear(dev_tensor(x), q.QuantWeight(dev_tensor(w), dev_tensor(s), dev_tensor(b)).tiled())
    torch.cuda.synchronize()
    ref = O.f64_to_bf16_bits(O.qlinear(x, w, s, b))
    np.testing.assert_array_equal(y.view(torch.uint16).cpu().numpy(), ref)


@pytest.mark.parametrize("M,N,K", [(37, 48, 192), (1, 16, 64), (100, 400, 320)])
def test_qlinear_ragged(M, N, K):
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[qlinear ragged] M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    W = synth.random_qtensor(rng, (N,), K)
    x = synth.make_activations(M, K, seed=3)
    y = q.qlinear(dev_tensor(x), dev_qweight(W).tiled())
    torch.cuda.synchronize()
    ref = O.qlinear(x, W.w, W.scales, W.biases)
    assert O.rowwise_rel_err(bf16_host(y), ref) <= 1e-2


def tiled_reference(w, s, b, split):
    """The tiled layout of include/qmoe.h (qmoe_tile_weight), built on the host
    from its definition: a pure rearrangement of codes, scales and biases."""
    E, rows, KW = w.shape
    G = KW // 8
    nblk = -(-split // 64) if split else -(-rows // 128)
    out = np.zeros((E, nblk, G, 4608), dtype=np.uint8)
    n = np.arange(16)
    for blk in range(nblk):
        for j in range(8):
            if split:
                c = 64 * blk + 16 * (j % 4) + n
                r = c if j < 4 else split + c
                ok = (c < split) & (r < rows)
            else:
                r = 128 * blk + 16 * j + n
                ok = r < rows
            rr = np.where(ok, r, 0)
            for q in range(4):  # lane L = 16 q + n: words 2q, 2q+1 of the group
                for t in range(2):
                    word = w[:, rr, :].reshape(E, 16, G, 8)[:, :, :, 2 * q + t].astype(np.uint64)
                    nib = [(word >> (4 * c)) & 0xF for c in range(8)]
                    new = sum(nib[2 * pp] << (4 * pp) for pp in range(4)) + \
                        sum(nib[2 * pp + 1] << (16 + 4 * pp) for pp in range(4))
                    new = np.where(ok[None, :, None], new, 0).astype(np.uint32)  # [E, 16, G]
                    i, half = j // 2, j % 2
                    off = 1024 * i + 16 * (16 * q + n) + 8 * half + 4 * t  # [16]
                    by = new.view(np.uint8).reshape(E, 16, G, 4)
                    for bb in range(4):  # advanced index first: [16, E, G]
                        out[:, blk, :, off + bb] = np.transpose(by[:, :, :, bb], (1, 0, 2))
            sv = np.where(ok[None, :, None], s[:, rr, :], 0).astype(np.uint32)
            bv = np.where(ok[None, :, None], b[:, rr, :], 0).astype(np.uint32)
            pair = (sv | (bv << 16)).astype(np.uint32).view(np.uint8).reshape(E, 16, G, 4)
            off = 4096 + 256 * (j // 4) + 16 * n + 4 * (j % 4)
            for bb in range(4):
                out[:, blk, :, off + bb] = np.transpose(pair[:, :, :, bb], (1, 0, 2))
    return out.reshape(-1)


@pytest.mark.parametrize("E,rows,K,split", [(3, 256, 192, 128), (2, 200, 128, 0), (1, 48, 64, 0),
                                           (2, 1408, 2816, 704), (1, 96, 128, 48), (2, 416, 64, 208)])
def test_tile_weight_layout_bitwise(E, rows, K, split):
    import bit_quantized_moe_diffrouter_amd as q
    say(f"[tile] E={E} rows={rows} K={K} split={split}")
    rng = np.random.default_rng(E * 1000 + rows + K)
    W = synth.random_qtensor(rng, (E, rows), K)
    t = dev_qweight(W).tiled(split)
    torch.cuda.synchronize()
    got = t.buf.cpu().numpy()
    ref = tiled_reference(W.w.reshape(E, rows, K // 8), W.scales.reshape(E, rows, K // 64),
                          W.biases.reshape(E, rows, K // 64), split)
    assert got.shape == ref.shape
    np.testing.assert_array_equal(got, ref)

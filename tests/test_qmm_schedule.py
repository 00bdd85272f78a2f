"""CPU emulation of the switch and dense kernels' schedules (qswitch.hip's
chunked kernel, qmm_tall.hip's gate_up launch and qmm_ws.hip's
weight-stationary pipeline).

The kernels' index arithmetic is restated here in Python, independently of
the device code: buckets and their two-tile and one-tile chunks, the
worker slots and their boustrophedon item order, the item decode (the
bucket search over the chunk prefixes), the activation tiles, the load
cursor running D units ahead of the compute cursor with its four-entry row
table (the down pass), and every address a load or store forms.  The tests
check, on the routings of the tiny, canvas, prefill and skewed workloads and
on the ragged layer shapes of the GPU tests, that:
  * every (item, contraction part) is computed by exactly one wave, and the
    waves of a worker walk the same items in the same order (so their
    partial-sum hand-over cannot deadlock);
  * the load cursor never enters item c + 4 while item c is being computed
    or finished (the row table entry of c is intact when its rows are
    stored);
  * every weight, activation, mid and output access lies inside its buffer;
  * the tall-tile kernel's gate_up launch (from 96 rows per expert) covers
    every (row chunk, block) of every expert exactly once, inside the
    buffers, and the weight-stationary kernel's per-group pipeline (register
    ring of codes and activations, two LDS buffers, one barrier per group)
    feeds every group's products with that group's operands.
No GPU is used."""
import numpy as np
import pytest

import oracle as O
import synth

NUM_CU = 256
KBM = 32
UNIT = 4608
ACT_BLOCK = 2048


def lds_bytes(mode, ks):
    wave = 2 * 16 * (64 if mode in ("gate_up", "dense_geglu") else 128) * 2
    return 4 * wave + (4 // ks) * (ks - 1) * 2 * 8 * 64 * 16


def max_items(mode, A, E, nblk):
    chunks = -(-A // KBM)
    if mode in ("gate_up", "down"):
        chunks += min(E, A) + (1 if mode == "down" else 0)
    return chunks * nblk


def choose_ks(mode, A, E, nblk, G):
    items = max_items(mode, A, E, nblk)
    four_fits = 2 * (lds_bytes(mode, 4) + 8192) <= 160 * 1024 or items <= NUM_CU
    ks = 2 if (mode == "gate_up" and G >= 8) else 1
    while ks < 4 and items * ks < 4 * NUM_CU and G >= 4 * ks and (ks == 1 or four_fits):
        ks *= 2
    return ks


def slot_of(worker, pos, workers, grid):
    return ((worker + pos) & (workers - 1)) * grid + pos


def emulate_chunked(mode, A, E, nblk, G, offsets=None, assign=None, T=None, ktop=None, Nout=None, K=None,
                    D=None, slot=slot_of):
    """One launch of the chunked kernel; raises AssertionError on a violated
    invariant, returns (KS, D, grid, items).  D and slot override the ring
    depth and the slot formula (for the planted-mistake tests)."""
    ks = choose_ks(mode, A, E, nblk, G)
    if D is None:
        D = 2 if (ks > 1 or G >= 2) else 1
    items_max = max_items(mode, A, E, nblk)
    grid = max(1, min(items_max, 2 * NUM_CU))
    rows_mode = mode == "dense"
    # ---- buckets and chunks
    if rows_mode:
        rem = A % KBM
        total2, total1 = A // KBM + (1 if rem > 16 else 0), (1 if 0 < rem <= 16 else 0)
    else:
        nb = E + 1 if mode == "down" else E
        lo, hi = np.zeros(nb, np.int64), np.zeros(nb, np.int64)
        c2, c1, tl = np.zeros(nb, np.int64), np.zeros(nb, np.int64), np.zeros(nb, np.int64)
        for b in range(nb):
            o0, o1 = int(offsets[b]), int(offsets[min(b + 1, E)])
            lo[b] = min(max(o0, 0), A)
            hi[b] = min(max(o1, lo[b]), A) if b < E else A
            n = hi[b] - lo[b]
            r = n % KBM
            c2[b] = n // KBM + (1 if r > 16 else 0)
            c1[b] = 1 if 0 < r <= 16 else 0
            tl[b] = -(-n // 16) if b < E else 0
        cum2 = np.concatenate([[0], np.cumsum(c2)])
        cum1 = np.concatenate([[0], np.cumsum(c1)])
        tcum = np.concatenate([[0], np.cumsum(tl)])
        total2, total1 = int(cum2[-1]), int(cum1[-1])
    max_tiles = -(-A // 16) + min(E, A)
    total_items = (total2 + total1) * nblk
    workers = 4 // ks
    nslots = grid * workers

    def decode(item):
        chunk = item // nblk
        blk = item - chunk * nblk
        if rows_mode:
            r0 = chunk * KBM
            return 0, r0, min(KBM, A - r0), blk, False
        two = chunk < total2
        c = chunk if two else chunk - total2
        cum = cum2 if two else cum1
        l, h = 0, nb
        while h - l > 1:
            mid = (l + h) >> 1
            if cum[mid] <= c:
                l = mid
            else:
                h = mid
        e = l
        assert cum[e] <= c < cum[e + 1], "bucket search landed outside the chunk's bucket"
        local = c - cum2[e] if two else cum2[e + 1] - cum2[e]
        r0 = int(lo[e] + local * KBM)
        rows = int(min(KBM, hi[e] - r0))
        zero = mode == "down" and e >= E
        assert 1 <= rows <= KBM and lo[e] <= r0 and r0 + rows <= hi[e]
        if two:
            assert rows > 16
        return (0 if zero else e), r0, rows, blk, zero

    def tile_of(e, r0, zero, m):
        if rows_mode or zero:
            return 0
        tau = int(tcum[e] + (r0 - lo[e]) // 16 + m)
        return tau if 0 <= tau < max_tiles else -1

    done = {}
    for b in range(grid):
        pos = (b % 8) * (grid // 8) + b // 8 if grid % 8 == 0 else b
        seqs = []
        for w in range(4):
            worker, kp = w // ks, w % ks
            gk0, gk1 = kp * G // ks, (kp + 1) * G // ks
            assert gk1 > gk0, "a wave with no groups"
            sl = slot(worker, pos, workers, grid)
            seq = []
            j = 0
            while True:
                item = j * nslots + (nslots - 1 - sl if j & 1 else sl)
                if item >= total_items:
                    break
                seq.append(item)
                j += 1
            seqs.append(seq)
            gw = gk1 - gk0
            for c, item in enumerate(seq):
                e, r0, rows, blk, zero = decode(item)
                key = (item, kp)
                assert key not in done, "an (item, part) computed twice"
                done[key] = True
                # the load cursor after the step of the item's last unit
                t_last = (c + 1) * gw - 1
                entered = min((t_last + D + 1) // gw, len(seq) - 1)
                assert entered <= c + 3, "the load cursor reached item c + 4 before item c was finished"
                # weights
                for g in range(gk0, gk1):
                    u = ((e * nblk + blk) * G + g)
                    assert 0 <= u < E * nblk * G if not rows_mode else 0 <= u < nblk * G
                # activations, per row tile m and half h
                for m in range(2):
                    mm = m if rows > 16 else 0
                    if mode == "down":
                        tau = max(tile_of(e, r0, zero, mm), 0)
                        assert tau < max_tiles
                        assert (tau * G + gk1 - 1) * ACT_BLOCK + 1024 + 1024 <= max_tiles * G * ACT_BLOCK
                    else:
                        for h in range(2):
                            rr = [min(16 * mm + 8 * h + (ln >> 3), rows - 1) for ln in range(64)]
                            if mode == "gate_up":
                                for x in rr:
                                    a = int(assign[r0 + x])
                                    src = a // ktop if 0 <= a < A else 0
                                    assert (src * K * 2 + (gk1 - 1) * 128 + 7 * 16 + 16) <= T * K * 2
                            else:
                                assert r0 + max(rr) < A
                # outputs (by the worker's first wave)
                if kp == 0:
                    for m in range(2 if rows > 16 else 1):
                        if mode == "gate_up":
                            tau = tile_of(e, r0, zero, m)
                            if tau >= 0:
                                assert (tau * (Nout // 64) + blk) * ACT_BLOCK + ACT_BLOCK <= max_tiles * (Nout // 64) * ACT_BLOCK
                        elif mode == "down":
                            for lr in range(16 * m, min(16 * m + 16, rows)):
                                a = int(assign[r0 + lr])
                                if 0 <= a < A:
                                    for col in range(blk * 128, min(blk * 128 + 128, Nout), 8):
                                        assert (a * Nout + col + 8) <= A * Nout
                        else:
                            assert r0 + min(16 * m + 16, rows) <= A
        for w in range(4):
            leader = (w // ks) * ks
            assert seqs[w] == seqs[leader], "the waves of a worker walk different items"
    for item in range(total_items):
        for kp in range(ks):
            assert (item, kp) in done, "an (item, part) never computed"
    return ks, D, grid, total_items


def emulate_tall_gate_up(A, E, nblk, G, offsets, assign, T, ktop, Nout, K, num_cu=NUM_CU, MT=8, NB=2, pos0_of=None):
    """The tall-tile gate_up launch: a persistent grid of at most one
    workgroup per compute unit, workgroup b starting at position pos0 (the
    workgroups numbered die by die) and stepping by the grid; position pos is
    chunk pos // nbp of the experts' 128-row chunks and the block pair
    pos % nbp (block 2 (pos % nbp) + wave // 2 for each wave).  Every
    (expert chunk, block) exactly once, inside the buffers.  pos0_of
    overrides the first position of a workgroup (for the planted-mistake
    test)."""
    BM = 16 * MT
    nbp = -(-nblk // NB)
    items = (-(-A // BM) + min(E, A)) * nbp
    grid = min(-(-items // 8) * 8, num_cu * (4 // (2 * NB)))
    lo = np.clip(offsets[:E], 0, A)
    hi = np.maximum(np.clip(offsets[1:E + 1], 0, A), lo)
    n = hi - lo
    cpre = np.concatenate([[0], np.cumsum(-(-n // BM))])
    tpre = np.concatenate([[0], np.cumsum(-(-n // 16))])
    max_tiles = -(-A // 16) + min(E, A)
    n_items = int(cpre[E]) * nbp
    assert n_items <= items
    NW, NS = 2 * NB, MT // (2 * NB)
    seen = set()
    for b in range(grid):
        pos0 = (b % 8) * (grid // 8) + b // 8 if grid % 8 == 0 else b
        if pos0_of is not None:
            pos0 = pos0_of(b, grid)
        for pos in range(pos0, n_items, grid):
            ch, bp = pos // nbp, pos % nbp
            e = int(np.count_nonzero(cpre[:E] <= ch)) - 1
            assert cpre[e] <= ch < cpre[e + 1]
            r0 = int(lo[e] + (ch - cpre[e]) * BM)
            rows = int(min(BM, hi[e] - r0))
            assert 1 <= rows and r0 + rows <= hi[e]
            tau0 = int(tpre[e] + (r0 - lo[e]) // 16)
            mt = -(-rows // 16)
            for wave in range(2 * NB):
                c, bsel = wave & 1, wave >> 1
                blk = bp * NB + bsel
                wblk = min(blk, nblk - 1)
                assert ((e * nblk + wblk) * G + G) * UNIT <= E * nblk * G * UNIT
                for s in range(NS):
                    for ln in range(16):
                        rl = min(16 * (wave + NW * s) + ln, rows - 1)
                        a = int(assign[r0 + rl])
                        src = a // ktop if 0 <= a < A else 0
                        assert src < T and src * K * 2 + (G - 1) * 128 + 3 * 32 + 32 <= T * K * 2
                if blk >= nblk:
                    continue
                if c == 0:
                    assert (e, r0, blk) not in seen, "an (expert chunk, block) computed twice"
                    seen.add((e, r0, blk))
                for m in range(mt):
                    tau = tau0 + m
                    if 0 <= tau < max_tiles:
                        last = (tau * (Nout // 64) + blk) * ACT_BLOCK + 1024 + 512 * c + 31 * 16 + 16
                        assert last <= max_tiles * (Nout // 64) * ACT_BLOCK
    expect = {(e, int(lo[e] + c * BM), blk) for e in range(E) for c in range(-(-int(n[e]) // BM)) for blk in range(nblk)}
    assert seen == expect, "an (expert chunk, block) never computed"


def emulate_ws_pipeline(G, PD, refill=None, ahead=None, prod_buf=None):
    """The weight-stationary kernel's per-group pipeline, step by step.  A
    ring slot holds one group's codes and scales and its activation operands;
    the prologue loads groups 0 .. PD-1 into slots 0 .. PD-1, dequantizes
    group 0 from slot 0 into LDS buffer 0, and reaches the barrier.  Step g
    (its slot d = g mod PD; the loop runs blocks of PD steps) dequantizes
    group g + 1 from slot (d + 1) mod PD into buffer (g + 1) mod 2, runs the
    products of group g from buffer g mod 2 with slot d's activations,
    refills slot d with group min(g + PD, G - 1), and reaches the barrier.
    Checks that every group's products read that group's dequantized
    weights and activations, once, in order, and that a step never writes
    the buffer its own products read (the other one was last read before
    the previous barrier).  refill, ahead and prod_buf override the slot the
    step refills, how far ahead it loads and the buffer the products read
    (for the planted-mistake tests)."""
    refill = refill or (lambda d, dn: d)
    ahead = PD if ahead is None else ahead
    prod_buf = prod_buf or (lambda g: g % 2)
    slots = [(min(d, G - 1), min(d, G - 1)) for d in range(PD)]  # (codes group, activations group)
    buf = [None, None]
    buf[0] = slots[0][0]
    done = []
    g = 0
    while g < G:
        for d in range(PD):
            if g >= G:
                break
            dn = (d + 1) % PD
            wrote = None
            if g + 1 < G:
                assert slots[dn][0] == g + 1, f"group {g + 1} dequantized from a slot holding {slots[dn][0]}"
                wrote = (g + 1) % 2
                buf[wrote] = g + 1
            b = prod_buf(g)
            assert wrote is None or wrote != b, "a step overwrites the buffer its products read"
            assert buf[b] == g, f"group {g}'s products read the weights of group {buf[b]}"
            assert slots[d][1] == g, f"group {g}'s products read the activations of group {slots[d][1]}"
            done.append(g)
            r = refill(d, dn)
            slots[r] = (min(g + ahead, G - 1), min(g + ahead, G - 1))
            g += 1
    assert done == list(range(G))


@pytest.mark.parametrize("PD", [2, 3])
def test_ws_pipeline(PD):
    for G in range(1, 50):
        emulate_ws_pipeline(G, PD)


def test_ws_pipeline_catches_planted_mistakes():
    """Refilling the slot just dequantized (group g + 1's) instead of group
    g's, loading one group less far ahead, and reading the products from the
    buffer being written all fail from 4 groups on."""
    for PD in (2, 3):
        with pytest.raises(AssertionError, match="slot holding|activations"):
            emulate_ws_pipeline(8, PD, refill=lambda d, dn: dn)
        with pytest.raises(AssertionError, match="slot holding|activations"):
            emulate_ws_pipeline(8, PD, ahead=PD - 1)
        with pytest.raises(AssertionError, match="overwrites|weights of"):
            emulate_ws_pipeline(8, PD, prod_buf=lambda g: (g + 1) % 2)


# ------------------------------------------------------------------ cases
_W = {}


def moe_inputs(cfg):
    if cfg.H == 2816:
        if "w" not in _W:
            _W["w"] = synth.make_moe_weights(synth.CANVAS)
        w = _W["w"]
        if cfg.zipf_tau is not None:
            w = synth.MoEWeights(w.norm_scale, w.router, w.per_expert_scale, w.gate_up, w.down,
                                 synth.zipf_logit_bias(cfg.E, cfg.zipf_tau, cfg.zipf_perm_seed))
        return synth.make_moe_inputs(cfg, w)
    return synth.make_moe_inputs(cfg)


def routing_of(cfg):
    inp = moe_inputs(cfg)
    wt = inp.weights
    r = wt.router
    idx, _, _ = O.route(inp.x, wt.norm_scale, cfg.eps, r.w, r.scales, r.biases, wt.per_expert_scale, cfg.k,
                        wt.logit_bias)
    return idx


def both_passes(idx, T, k, E, H, I):
    off, sa = O.sort_assignments(np.where((idx >= 0) & (idx < E), idx, E), E)
    flat = np.asarray(idx).reshape(-1)
    # moe_sort drops out-of-range indices into a tail bucket after offsets[E]
    order = np.argsort(np.where((flat >= 0) & (flat < E), flat, E), kind="stable").astype(np.int64)
    A = T * k
    ks_g = emulate_chunked("gate_up", A, E, -(-I // 64), H // 64, off, order, T, k, I, H)
    ks_d = emulate_chunked("down", A, E, -(-H // 128), I // 64, off, order, T, k, H, I)
    if A >= 96 * E:
        emulate_tall_gate_up(A, E, -(-I // 64), H // 64, off, order, T, k, I, H)
    return ks_g, ks_d


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [synth.TINY, synth.CANVAS, synth.SKEW, synth.PREFILL], ids=lambda c: c.name)
def test_chunked_schedule_on_workload_routings(cfg):
    idx = routing_of(cfg)
    both_passes(idx, cfg.T, cfg.k, cfg.E, cfg.H, cfg.I)


@pytest.mark.parametrize("T,H,E,k,I", [(1, 64, 1, 1, 64), (37, 192, 12, 3, 192), (9, 256, 8, 8, 64),
                                       (45, 576, 12, 4, 320), (200, 512, 6, 4, 128), (40, 128, 256, 16, 64),
                                       (300, 256, 5, 2, 320), (1000, 128, 1, 1, 64), (250, 192, 16, 8, 192)])
def test_chunked_schedule_on_ragged_layers(T, H, E, k, I):
    cfg = synth.MoEConfig("ragged", T=T, H=H, E=E, k=k, I=I, seed_w=31, seed_x=32)
    both_passes(routing_of(cfg), T, k, E, H, I)


def test_chunked_schedule_with_dropped_and_hot_experts():
    rng = np.random.default_rng(5)
    T, k, E, H, I = 256, 8, 128, 2816, 704
    idx = rng.integers(0, E, size=(T, k))
    idx[rng.random((T, k)) < 0.5] = 7      # one hot expert
    idx[rng.random((T, k)) < 0.03] = -1    # dropped
    idx[0, 0] = E
    both_passes(idx, T, k, E, H, I)


@pytest.mark.parametrize("M,K,N", [(2520, 1152, 1152), (1, 64, 64), (17, 192, 128), (100, 1152, 2064),
                                   (256, 2816, 4224)])
def test_dense_schedule(M, K, N):
    emulate_chunked("dense", M, 1, -(-N // 128), K // 64)


def test_emulation_catches_planted_mistakes():
    """The checks fire on a broken slot formula (two workers on the same
    items: some computed twice, others never) and on a ring deep enough to
    reach item c + 4 before item c is finished (one group per wave)."""
    with pytest.raises(AssertionError, match="twice|never"):
        emulate_chunked("dense", 2520, 1, 9, 18, slot=lambda worker, pos, workers, grid: pos)
    # one group per wave and about five items per wave: the kernel's ring of
    # one slot passes, a ring of four would overwrite item c's row entry
    emulate_chunked("dense", 40000, 1, 8, 1)
    with pytest.raises(AssertionError, match="c \\+ 4"):
        emulate_chunked("dense", 40000, 1, 8, 1, D=4)


def test_tall_gate_up_emulation_catches_planted_mistakes():
    """Dropping the per-die index from the first position (every workgroup of
    a die then starts on the same item) computes some items twice and others
    never."""
    T, k, E, H, I = 1024, 8, 16, 256, 704
    idx = np.random.default_rng(9).integers(0, E, size=(T, k))
    off, _ = O.sort_assignments(idx, E)
    order = np.argsort(idx.reshape(-1), kind="stable").astype(np.int64)
    args = (T * k, E, -(-I // 64), H // 64, off, order, T, k, I, H)
    emulate_tall_gate_up(*args)
    with pytest.raises(AssertionError, match="twice|never"):
        emulate_tall_gate_up(*args, pos0_of=lambda b, grid: (b % 8) * (grid // 8))

"""Plain CPU oracle for the 4-bit group-quantized mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Sources.  The pages are three diff-viewer pages of the npm package
"@mlx-bun/inference 0.0.0-stage -> 1.0.0".  Citations below name the page by
the source file it shows and the class / method the passage sits in:

* [model page]   package/src/models/diffusion-gemma/model.ts
* [vision page]  package/src/models/diffusion-gemma/vision.ts
* [assistant page] package/src/models/gemma4/assistant.ts

What is computed, step by step (fp64 unless stated):

Q  unpack + dequantize a 4-bit affine weight: ``W = scale * q + bias`` per
   64-wide group                  ([model page] dequantEmbedWeight; the packed
   uint32 weight of a quantized linear: [vision page] VisionLinear.weightDtype)
R1 RMSNormNoScale ``x / sqrt(mean(x^2) + eps)``
                                  ([vision page] manualRms with a null weight;
                                   [model page] DiffRouter.forward)
R2 ``u = r * scale[h] * H^-0.5`` as separate multiplies after the norm
                                  ([model page] DiffRouter comment + forward)
R3 logits ``u . W_r^T`` (+ optional per-expert offset), stored fp32
                                  ([model page] DiffRouter.forward, proj)
R4 top-k experts, descending, ties to the lower expert index
                                  ([model page] DiffRouter.forward, argpartition;
                                   tie rule read from [assistant page] centroid head)
R5 precise softmax over the k gathered logits, times per_expert_scale[idx]
                                  ([model page] DiffRouter.forward)
S  token-by-expert sort: stable order of assignment ids a = t*k + j by expert
                                  ([model page] DiffExperts.forward, argsort)
X  per assignment: ``g = x_t . W_gu[e]^T``, split at I, ``gelu_tanh(gate) * up``,
   ``d = mid . W_d[e]^T``; per token ``y_t = sum_j w_tj d_tj``
                                  ([model page] DiffExperts.forward; GeGLU as
                                   gelu_approx(gate) * up: [vision page] DiffVisionMLP)
L  dense 4-bit linear ``y = x . W^T``
                                  ([vision page] VisionLinear.forward, quantized arm)
H  the tied LM head: ``cap * tanh(bf16(x . E^T) / cap)``, fp32 out
                                  ([model page] logitsFromHidden, the softcap
                                   default in the constructor)
C  self-conditioning embedding: ``bf16(bf16(softmax(z) . E) * embed_scale)``
   with the table E used without transposing
                                  ([model page] #embedCanvas)
F  the decoder's feed-forward block around the MoE: plain RMSNorm with its
   weight used as stored (no 1 + w offset); the parallel dense GeGLU MLP
   ``down(gelu_tanh(gate x) * up x)``; ``out = (h + N(N1(h1) + N2(h2))) * s``
   with h1 the dense branch on N0(h), h2 the experts on N0'(h), the router
   on the raw h                   ([model page] DiffDecoderLayer.forwardWith,
                                   the file header's note on plain RMSNorm;
                                   the MLP shape: SelfConditioning, GegluMLP)

Readings where the pages are silent: group 64,
codes stored first-in-lowest-bits, scales/biases bf16; eps = 1e-6; router kept
in fp32/fp64 without the pages' intermediate bf16 roundings; ties to the lower
expert index; stable sort; tanh-form GELU.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

GROUP = 64


# ----------------------------------------------------------------------------
# storage decoding (bf16 is carried as its uint16 bit pattern)
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns: the pattern is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round to bfloat16, nearest-even, via fp32 (for reporting outputs only)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ----------------------------------------------------------------------------
# Q: 4-bit affine group quantization
# ----------------------------------------------------------------------------
def unpack_codes(words: np.ndarray) -> np.ndarray:
    """Packed uint32 words [..., K/8] -> codes uint8 [..., K].

    Code c of a row sits in word c // 8 at bits 4*(c % 8) .. 4*(c % 8) + 3
    (first code in the lowest bits).  The pages show the packed weight as a
    uint32 array ([vision page] VisionLinear.weightDtype) but not the field
    order; this reading is pinned by a golden file.
    """
    w = np.asarray(words, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32)).reshape((1,) * w.ndim + (8,))
    q = (w[..., None] >> shifts) & np.uint32(0xF)
    return q.reshape(w.shape[:-1] + (w.shape[-1] * 8,)).astype(np.uint8)


def dequantize(words, scales, biases, group: int = GROUP) -> np.ndarray:
    """``W[n, c] = scale[n, c // group] * q[n, c] + bias[n, c // group]`` in fp64
    ([model page] dequantEmbedWeight: dequantize(w, scales, biases))."""
    q = unpack_codes(words).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), group, axis=-1)
    b = np.repeat(bf16_to_f64(biases), group, axis=-1)
    assert q.shape == s.shape == b.shape, (q.shape, s.shape)
    return s * q + b


def dequantize_f32(words, scales, biases, group: int = GROUP) -> np.ndarray:
    """The same dequantization evaluated in fp32 (used by the grouped path)."""
    q = unpack_codes(words).astype(np.float32)
    s = np.repeat(bf16_to_f64(scales).astype(np.float32), group, axis=-1)
    b = np.repeat(bf16_to_f64(biases).astype(np.float32), group, axis=-1)
    return s * q + b


# ----------------------------------------------------------------------------
# L: dense 4-bit linear
# ----------------------------------------------------------------------------
def qlinear(x_bits, words, scales, biases) -> np.ndarray:
    """``y = x . dequant(W)^T`` accumulated in fp64 ([vision page]
    VisionLinear.forward; the quantized matmul multiplies by the transposed
    weight by default, [model page] #embedCanvas passes transpose=false only
    for the embedding)."""
    x = bf16_to_f64(x_bits)
    W = dequantize(words, scales, biases)
    return x @ W.T


# ----------------------------------------------------------------------------
# R: router
# ----------------------------------------------------------------------------
def rms_norm_noscale(x: np.ndarray, eps: float) -> np.ndarray:
    """R1: ``x / sqrt(mean(x^2) + eps)`` over the last axis ([vision page]
    manualRms with weight = null is the NoScale form)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def router_prologue(x_bits, norm_scale_bits, eps: float) -> np.ndarray:
    """R1 + R2: ``u = rms_norm_noscale(x) * scale * H^-0.5`` ([model page]
    DiffRouter.forward: norm, then times scale, then times rootSize).
    H^-0.5 is formed in double and rounded to fp32, as the pages' rootSize is a
    double handed to a float multiply."""
    x = bf16_to_f64(x_bits)
    H = x.shape[-1]
    root = float(np.float32(math.pow(H, -0.5)))
    return rms_norm_noscale(x, eps) * bf16_to_f64(norm_scale_bits) * root


def router_logits(u: np.ndarray, proj_w, proj_s, proj_b,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """R3: ``logits = u . dequant(W_r)^T (+ offset)``, fp64 accumulate, stored fp32."""
    Wr = dequantize(proj_w, proj_s, proj_b)
    logits = u @ Wr.T
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)
    return logits.astype(np.float32)


def top_k(logits: np.ndarray, k: int) -> np.ndarray:
    """R4: indices of the k largest logits per row, in descending order of
    logit, ties to the lower expert index (a stable sort of the negated
    logits keeps equal values in index order)."""
    order = np.argsort(-np.asarray(logits, dtype=np.float64), axis=-1, kind="stable")
    return order[..., :k].astype(np.int32)


def precise_softmax(v: np.ndarray) -> np.ndarray:
    """R5: ``exp(v - max) / sum(exp(v - max))`` over the last axis in fp64
    ([model page] softmaxAxis(w, -1, precise = true))."""
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(v - v.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def route(x_bits, norm_scale_bits, eps: float, proj_w, proj_s, proj_b,
          pes_bits, k: int, logit_bias: Optional[np.ndarray] = None
          ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The DiffRouter ([model page] DiffRouter.forward):
    x [T, H] -> (indices int32 [T, k], weights fp32 [T, k], logits fp32 [T, E]).

    The softmax runs over the fp32 logits as stored; the weights are
    ``p_j * per_expert_scale[e_j]`` rounded to fp32."""
    u = router_prologue(x_bits, norm_scale_bits, eps)
    logits = router_logits(u, proj_w, proj_s, proj_b, logit_bias)
    idx = top_k(logits, k)
    picked = np.take_along_axis(logits.astype(np.float64), idx, axis=-1)
    p = precise_softmax(picked)
    w = p * bf16_to_f64(pes_bits)[idx]
    return idx, w.astype(np.float32), logits


def gap_kth(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row: the k-th largest logit minus the (k+1)-th (inf when k = E)."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=-1)
    if k >= s.shape[-1]:
        return np.full(s.shape[:-1], np.inf)
    return s[..., k - 1] - s[..., k]


# ----------------------------------------------------------------------------
# S: sort
# ----------------------------------------------------------------------------
def sort_assignments(indices: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """S ([model page] DiffExperts.forward: order = argsort(flat idx)).

    Returns ``expert_offsets`` int32 [E + 1] (exclusive prefix sum of the
    per-expert counts) and ``sorted_assign`` int32 [T * k]: assignment ids
    ``a = t * k + j`` grouped by expert, ascending within an expert (stable)."""
    flat = np.asarray(indices, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")
    return offsets.astype(np.int32), order.astype(np.int32)


# ----------------------------------------------------------------------------
# X: experts
# ----------------------------------------------------------------------------
def gelu_tanh(z):
    """Tanh-form GELU: ``0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))``
    ([vision page] DiffVisionMLP uses gelu_approx(gate) * up)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def expert_rows_bruteforce(x_row: np.ndarray, e: int, gate_up, down, I: int
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """One assignment, fp64: returns (mid [I], d [H]) for token row x_row
    (fp64 [H]) routed to expert e ([model page] DiffExperts.forward:
    gate_up, split at moe_intermediate, geglu, down)."""
    Wgu = dequantize(gate_up.w[e], gate_up.scales[e], gate_up.biases[e])
    Wd = dequantize(down.w[e], down.scales[e], down.biases[e])
    g = Wgu @ x_row
    mid = gelu_tanh(g[:I]) * g[I:]
    return mid, Wd @ mid


def _as_f64(x) -> np.ndarray:
    """bf16 bit patterns (uint16) are decoded; anything else is taken as values."""
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def experts_bruteforce(x_bits, indices, weights, gate_up, down, I: int,
                       tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """X by brute force, per token and per slot in fp64, no sort:
    ``y_t = sum_j w_tj * down_e(geglu(gate_up_e(x_t)))`` summed in j order
    ([model page] DiffExperts.forward, final weighted sum over k).

    ``tokens`` restricts the computation to those rows (returned in that
    order).  Each touched expert is dequantized once.  ``x_bits`` may also be
    an array of values (the feed-forward block passes a norm's output)."""
    x = _as_f64(x_bits)
    idx = np.asarray(indices)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    T, k = idx.shape
    toks = list(range(T)) if tokens is None else list(tokens)
    need = sorted({int(idx[t, j]) for t in toks for j in range(k)})
    H = x.shape[1]
    y = np.zeros((len(toks), H))
    contrib = {}
    for e in need:
        Wgu = dequantize(gate_up.w[e], gate_up.scales[e], gate_up.biases[e])
        Wd = dequantize(down.w[e], down.scales[e], down.biases[e])
        for ti, t in enumerate(toks):
            for j in range(k):
                if int(idx[t, j]) == e:
                    g = Wgu @ x[t]
                    mid = gelu_tanh(g[:I]) * g[I:]
                    contrib[(ti, j)] = Wd @ mid
    for ti, t in enumerate(toks):
        for j in range(k):
            y[ti] += w[t, j] * contrib[(ti, j)]
    return y


def expert_mid_bruteforce(x_bits, indices, gate_up, I: int,
                          assignments: Sequence[int]) -> np.ndarray:
    """``mid`` (fp64 [len(assignments), I]) for the given assignment ids
    a = t * k + j, computed per assignment."""
    x = bf16_to_f64(x_bits)
    idx = np.asarray(indices)
    k = idx.shape[1]
    out = np.zeros((len(assignments), I))
    by_e = {}
    for i, a in enumerate(assignments):
        by_e.setdefault(int(idx[a // k, a % k]), []).append((i, a))
    for e, items in by_e.items():
        Wgu = dequantize(gate_up.w[e], gate_up.scales[e], gate_up.biases[e])
        for i, a in items:
            g = Wgu @ x[a // k]
            out[i] = gelu_tanh(g[:I]) * g[I:]
    return out


def down_combine_from_mid(mid_rows: np.ndarray, indices, weights, down,
                          tokens: Sequence[int]) -> np.ndarray:
    """Down projection plus the weighted sum over k, starting from given
    per-assignment ``mid`` rows (``mid_rows[a]`` for assignment a = t*k + j).
    fp64, summed in j order."""
    idx = np.asarray(indices)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    k = idx.shape[1]
    mid = np.asarray(mid_rows, dtype=np.float64)
    H = down.w.shape[1]
    y = np.zeros((len(tokens), H))
    cache = {}
    for ti, t in enumerate(tokens):
        for j in range(k):
            e = int(idx[t, j])
            if e not in cache:
                cache[e] = dequantize(down.w[e], down.scales[e], down.biases[e])
            y[ti] += w[t, j] * (cache[e] @ mid[t * k + j])
    return y


def experts_grouped(x_bits, indices, weights, gate_up, down, I: int) -> np.ndarray:
    """X the grouped way, fp32 throughout: sort the assignments by expert (S),
    then per touched expert dequantize its two weights and run two fp32
    matmuls over its rows, then the weighted sum over k in j order.  Same
    definition as experts_bruteforce; this is the form timed as the CPU
    baseline."""
    x = bf16_to_f64(x_bits).astype(np.float32)
    idx = np.asarray(indices)
    w = np.asarray(weights, dtype=np.float32)
    T, k = idx.shape
    E = gate_up.w.shape[0]
    offsets, order = sort_assignments(idx, E)
    d = np.zeros((T * k, x.shape[1]), dtype=np.float32)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        a = order[lo:hi]
        xs = x[a // k]
        Wgu = dequantize_f32(gate_up.w[e], gate_up.scales[e], gate_up.biases[e])
        Wd = dequantize_f32(down.w[e], down.scales[e], down.biases[e])
        g = xs @ Wgu.T
        mid = (gelu_tanh(g[:, :I]) * g[:, I:]).astype(np.float32)
        d[a] = mid @ Wd.T
    y = np.zeros((T, x.shape[1]), dtype=np.float32)
    for j in range(k):
        y += w[:, j:j + 1] * d[j::k]
    return y


def moe_layer(x_bits, weights, k: int, I: int, eps: float, grouped: bool = True):
    """The whole layer: route, then experts.  Returns (y, indices, weights, logits)."""
    r = weights.router
    idx, wts, logits = route(x_bits, weights.norm_scale, eps, r.w, r.scales, r.biases,
                             weights.per_expert_scale, k, weights.logit_bias)
    if grouped:
        y = experts_grouped(x_bits, idx, wts, weights.gate_up, weights.down, I)
    else:
        y = experts_bruteforce(x_bits, idx, wts, weights.gate_up, weights.down, I)
    return y, idx, wts, logits


# ----------------------------------------------------------------------------
# F: the decoder's feed-forward block
# ----------------------------------------------------------------------------
def rms_norm(x, weight_bits, eps: float) -> np.ndarray:
    """Plain RMSNorm, ``x / sqrt(mean(x^2) + eps) * w`` over the last axis, the
    stored weight used as is ([model page] header: plain RMSNorm everywhere,
    no 1 + weight offset; [vision page] manualRms with a weight)."""
    return rms_norm_noscale(_as_f64(x), eps) * bf16_to_f64(weight_bits)


def dense_geglu(x, gate, up, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """First half of the dense branch, ``gelu_tanh(gate . x) * (up . x)``, fp64."""
    x = _as_f64(x)
    if rows is not None:
        x = x[list(rows)]
    g = x @ dequantize(gate.w, gate.scales, gate.biases).T
    u = x @ dequantize(up.w, up.scales, up.biases).T
    return gelu_tanh(g) * u


def dense_geglu_mlp(x, gate, up, down, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The dense branch ``down(gelu_tanh(gate . x) * (up . x))`` with three 4-bit
    linears, fp64 ([model page] DiffDecoderLayer's GegluMLP, the same shape as
    SelfConditioning's down(geglu(gate(.), up(.))); GeGLU as in the experts)."""
    return dense_geglu(x, gate, up, rows) @ dequantize(down.w, down.scales, down.biases).T


def ff_block(h_bits, moe_weights, ffw, k: int, I: int, eps: float,
             tokens: Optional[Sequence[int]] = None, route_out=None):
    """The feed-forward half of a decoder layer, fp64 with no intermediate
    rounding ([model page] DiffDecoderLayer.forwardWith, after the attention
    residual):

        residual = h
        h1 = postFfNorm1(mlp(preFfNorm(h)))
        (indices, weights) = router(h)                 # on the raw residual
        h2 = postFfNorm2(experts(preFfNorm2(h), indices, weights))
        out = (residual + postFfNorm(h1 + h2)) * layer_scalar

    ``tokens`` restricts the output rows (routing is per token, so only those
    tokens are routed); ``route_out`` = (indices, weights) replaces the
    oracle's own routing.  Returns (out [len(tokens), H], indices, weights)."""
    h = bf16_to_f64(h_bits)
    toks = list(range(h.shape[0])) if tokens is None else list(tokens)
    if route_out is None:
        r = moe_weights.router
        idx, wts, _ = route(np.asarray(h_bits)[toks], moe_weights.norm_scale, eps, r.w, r.scales, r.biases,
                            moe_weights.per_expert_scale, k, moe_weights.logit_bias)
    else:
        idx, wts = (np.asarray(route_out[0])[toks], np.asarray(route_out[1])[toks])
    hs = h[toks]
    h1 = rms_norm(dense_geglu_mlp(rms_norm(hs, ffw.pre_ff, eps), ffw.gate, ffw.up, ffw.down), ffw.post_ff1, eps)
    xe = rms_norm(hs, ffw.pre_ff2, eps)
    h2 = rms_norm(experts_bruteforce(xe, idx, wts, moe_weights.gate_up, moe_weights.down, I), ffw.post_ff2, eps)
    out = (hs + rms_norm(h1 + h2, ffw.post_ff, eps)) * ffw.layer_scalar
    return out, idx, wts


# ----------------------------------------------------------------------------
# H: the tied LM head and its softcap
# ----------------------------------------------------------------------------
def softcap(z, cap: float) -> np.ndarray:
    """``cap * tanh(z / cap)`` in fp64 ([model page] logitsFromHidden: a tanh
    softcap of the fp32-widened logits, cap = finalLogitSoftcapping, 30 when
    the config leaves it out)."""
    z = np.asarray(z, dtype=np.float64)
    return cap * np.tanh(z / cap)


def lm_head_softcap(x_bits, words, scales, biases, cap: float,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The tied head ([model page] logitsFromHidden): the embedding's 4-bit
    weight used as a linear, ``z = x . dequant(E)^T``, returned in the input's
    dtype (bf16, rounded to nearest even) as the quantized matmul returns it,
    then widened and softcapped.  ``rows`` restricts the output rows."""
    x = bf16_to_f64(x_bits)
    if rows is not None:
        x = x[list(rows)]
    z = x @ dequantize(words, scales, biases).T
    return softcap(bf16_to_f64(f64_to_bf16_bits(z)), cap)


# ----------------------------------------------------------------------------
# C: the self-conditioning embedding (probabilities times the embedding table)
# ----------------------------------------------------------------------------
def softmax_rows_bf16(logits) -> np.ndarray:
    """Precise softmax over the last axis in fp64, cast to bf16 bit patterns
    ([model page] #embedCanvas: softmaxAxis(scLogits, -1, precise) then
    astype to the embeddings' dtype)."""
    return f64_to_bf16_bits(precise_softmax(logits))


def embed_matmul_t(probs_bits, words, scales, biases, scale: float,
                   rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """``bf16(bf16(p . dequant(E)) * scale)`` with E the embedding table
    [V, H] used without transposing ([model page] #embedCanvas: the quantized
    matmul with transpose = false returns bf16, then mulScalar by embed_scale):
    probabilities [L, V] bf16 -> [L, H], fp64 inside each step.  ``rows``
    restricts the output rows."""
    p = bf16_to_f64(probs_bits)
    if rows is not None:
        p = p[list(rows)]
    se = bf16_to_f64(f64_to_bf16_bits(p @ dequantize(words, scales, biases)))
    return bf16_to_f64(f64_to_bf16_bits(se * np.float64(np.float32(scale))))


# ----------------------------------------------------------------------------
# error metric used by the parity tests
# ----------------------------------------------------------------------------
def rowwise_rel_err(y, ref) -> float:
    """``max_t max_h |y - ref| / max_h |ref|`` (per-row normalised max error)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(y - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max()) if num.size else 0.0

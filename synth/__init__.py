"""Seeded synthetic inputs for the 4-bit mixture-of-experts layer and the dense
4-bit linear.

This module is shared by the oracle tests, the GPU tests and the benchmark.  It
holds none of the layer's arithmetic: it only draws random numbers, rounds them
to bfloat16 storage, and hands out the packed 4-bit weight format as random
32-bit words (every 4-bit field of a uniform 32-bit word is itself uniform on
0..15 and independent of the others, so a uniform word *is* eight uniform
codes packed together, whatever the field order).

Workload recipe (one line per tensor, in draw order of the weight stream):

* router norm scale ``s[h] ~ U[0.8, 1.2]``                     -> bf16 ``[H]``
* router projection codes                                        -> u32  ``[E, H/8]``
* router projection scales ``|N(0, 0.02)|``, biases ``-8*scale`` -> bf16 ``[E, H/64]``
  (or, with a bias seed, biases drawn independently of the scales from a
  stream of their own: ``bf16(-scale * U[6, 9.5] + N(0, 0.01))``, so that a
  kernel which derived the bias from the scale would be caught)
* ``per_expert_scale ~ U[0.5, 1.5]``                            -> bf16 ``[E]``
* gate_up codes / scales / biases                                -> ``[E, 2I, H/8]`` / ``[E, 2I, H/64]``
* down codes / scales / biases                                   -> ``[E, H, I/8]`` / ``[E, H, I/64]``

The activations come from an independent stream: ``x ~ N(0, 1)`` -> bf16 ``[T, H]``.

The decoder's feed-forward block (MoE plus the parallel dense GeGLU branch)
adds, from a stream of its own: the five RMSNorm weights ``~ U[0.8, 1.2]``
(pre, pre_2, post_1, post_2, post) -> bf16 ``[H]``; the dense gate, up and down
4-bit weights (same recipe as above) ``[I_d, H/8]``, ``[I_d, H/8]``,
``[H, I_d/8]``; and ``layer_scalar ~ U[0.5, 1.5]`` rounded to bf16.
The skewed-routing workload adds a per-expert logit offset
``tau * ln p_e`` with ``p_e`` proportional to ``rank_e ** -1.1`` (Zipf, s = 1.1)
and ``rank`` a seeded permutation of ``1..E``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GROUP = 64


# ----------------------------------------------------------------------------
# storage helpers (bfloat16 is carried as its uint16 bit pattern)
# ----------------------------------------------------------------------------
def to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_as_f32(b) -> np.ndarray:
    """bfloat16 bit pattern -> fp32 value (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 2**32, size=shape, dtype=np.uint32)


def _scales_biases(rng: np.random.Generator, shape, bias_rng: Optional[np.random.Generator] = None):
    scales = to_bf16_bits(np.abs(rng.normal(0.0, 0.02, size=shape)).astype(np.float32))
    if bias_rng is None:
        # -8 * scale is exact in bfloat16 (power-of-two multiply, sign flip)
        biases = to_bf16_bits(-8.0 * bf16_bits_as_f32(scales))
    else:
        u = bias_rng.uniform(6.0, 9.5, size=shape)
        n = bias_rng.normal(0.0, 0.01, size=shape)
        biases = to_bf16_bits((-bf16_bits_as_f32(scales) * u + n).astype(np.float32))
    return scales, biases


@dataclass
class QTensor:
    """A 4-bit affine group-quantized weight: ``w`` packed codes (uint32,
    ``[..., rows, in/8]``), ``scales`` and ``biases`` (bf16 bits,
    ``[..., rows, in/64]``)."""

    w: np.ndarray
    scales: np.ndarray
    biases: np.ndarray

    @property
    def in_features(self) -> int:
        return self.w.shape[-1] * 8

    @property
    def rows(self) -> int:
        return self.w.shape[-2]

    @property
    def experts(self) -> int:
        return 1 if self.w.ndim == 2 else self.w.shape[0]

    @property
    def nbytes(self) -> int:
        return self.w.nbytes + self.scales.nbytes + self.biases.nbytes


def random_qtensor(rng: np.random.Generator, lead_shape, in_features: int,
                   bias_rng: Optional[np.random.Generator] = None) -> QTensor:
    assert in_features % GROUP == 0
    w = _codes(rng, tuple(lead_shape) + (in_features // 8,))
    s, b = _scales_biases(rng, tuple(lead_shape) + (in_features // GROUP,), bias_rng)
    return QTensor(w, s, b)


def _bias_rng(seed: Optional[int]) -> Optional[np.random.Generator]:
    return None if seed is None else np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    seed_w: int
    seed_x: int
    zipf_tau: Optional[float] = None
    zipf_perm_seed: int = 4
    eps: float = 1e-6
    bias_seed: Optional[int] = None   # set: biases independent of the scales


@dataclass(frozen=True)
class QLinearConfig:
    name: str
    M: int
    N: int
    K: int
    seed_w: int
    seed_x: int
    bias_seed: Optional[int] = None


TINY = MoEConfig("tiny_16tok_h256_e8_top2", T=16, H=256, E=8, k=2, I=128, seed_w=0, seed_x=0)
QLINEAR_VISION = QLinearConfig("qlinear_2520x1152_to_1152", M=2520, N=1152, K=1152, seed_w=1, seed_x=1)
CANVAS = MoEConfig("moe_canvas_256tok_h2816_e128_top8", T=256, H=2816, E=128, k=8, I=704,
                   seed_w=2, seed_x=2)
PREFILL = MoEConfig("moe_prefill_4096tok_h2816_e128_top8", T=4096, H=2816, E=128, k=8, I=704,
                    seed_w=2, seed_x=3)
SKEW = MoEConfig("moe_canvas_skew_256tok_zipf1.1", T=256, H=2816, E=128, k=8, I=704,
                 seed_w=2, seed_x=2, zipf_tau=0.1)

# decode-sized batches on the canvas weights: the unsorted arm's regime (T*k < 64)
DECODE_1 = MoEConfig("moe_decode_1tok_h2816_e128_top8", T=1, H=2816, E=128, k=8, I=704, seed_w=2, seed_x=5)
DECODE_7 = MoEConfig("moe_decode_7tok_h2816_e128_top8", T=7, H=2816, E=128, k=8, I=704, seed_w=2, seed_x=6)

CONFIGS = {c.name: c for c in (TINY, QLINEAR_VISION, CANVAS, PREFILL, SKEW, DECODE_1, DECODE_7)}


@dataclass
class MoEWeights:
    norm_scale: np.ndarray           # bf16 bits [H]
    router: QTensor                  # [E, H/8]
    per_expert_scale: np.ndarray     # bf16 bits [E]
    gate_up: QTensor                 # [E, 2I, H/8]
    down: QTensor                    # [E, H, I/8]
    logit_bias: Optional[np.ndarray] = None  # fp32 [E]

    @property
    def nbytes(self) -> int:
        n = self.norm_scale.nbytes + self.router.nbytes + self.per_expert_scale.nbytes
        return n + self.gate_up.nbytes + self.down.nbytes


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: np.ndarray                    # bf16 bits [T, H]
    weights: MoEWeights = field(repr=False)


def zipf_logit_bias(E: int, tau: float, perm_seed: int, s: float = 1.1) -> np.ndarray:
    rank = np.random.default_rng(perm_seed).permutation(E) + 1
    p = rank.astype(np.float64) ** (-s)
    p /= p.sum()
    return (tau * np.log(p)).astype(np.float32)


def make_moe_weights(cfg: MoEConfig, seed: Optional[int] = None) -> MoEWeights:
    rng = np.random.default_rng(cfg.seed_w if seed is None else seed)
    brng = _bias_rng(cfg.bias_seed)
    H, E, I = cfg.H, cfg.E, cfg.I
    norm_scale = to_bf16_bits(rng.uniform(0.8, 1.2, size=H).astype(np.float32))
    router = random_qtensor(rng, (E,), H, brng)
    pes = to_bf16_bits(rng.uniform(0.5, 1.5, size=E).astype(np.float32))
    gate_up = random_qtensor(rng, (E, 2 * I), H, brng)
    down = random_qtensor(rng, (E, H), I, brng)
    bias = None
    if cfg.zipf_tau is not None:
        bias = zipf_logit_bias(E, cfg.zipf_tau, cfg.zipf_perm_seed)
    return MoEWeights(norm_scale, router, pes, gate_up, down, bias)


def make_activations(T: int, H: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal(size=(T, H), dtype=np.float32))


def make_moe_inputs(cfg: MoEConfig, weights: Optional[MoEWeights] = None) -> MoEInputs:
    if weights is None:
        weights = make_moe_weights(cfg)
    return MoEInputs(cfg, make_activations(cfg.T, cfg.H, cfg.seed_x), weights)


@dataclass
class QLinearInputs:
    cfg: QLinearConfig
    x: np.ndarray      # bf16 bits [M, K]
    W: QTensor         # [N, K/8]


def make_qlinear_inputs(cfg: QLinearConfig) -> QLinearInputs:
    rng = np.random.default_rng(cfg.seed_w)
    W = random_qtensor(rng, (cfg.N,), cfg.K, _bias_rng(cfg.bias_seed))
    return QLinearInputs(cfg, make_activations(cfg.M, cfg.K, cfg.seed_x), W)


# ----------------------------------------------------------------------------
# the decoder's feed-forward block: MoE + parallel dense GeGLU MLP
# ----------------------------------------------------------------------------
@dataclass
class FFConfig:
    name: str
    moe: MoEConfig
    I_dense: int       # width of the dense GeGLU branch (not printed by the pages)
    seed_ff: int


@dataclass
class FFWeights:
    pre_ff: np.ndarray      # bf16 bits [H]: norm before the dense branch
    pre_ff2: np.ndarray     # bf16 bits [H]: norm before the experts
    post_ff1: np.ndarray    # bf16 bits [H]: norm after the dense branch
    post_ff2: np.ndarray    # bf16 bits [H]: norm after the experts
    post_ff: np.ndarray     # bf16 bits [H]: norm of the sum
    gate: QTensor           # [I_d, H/8]
    up: QTensor             # [I_d, H/8]
    down: QTensor           # [H, I_d/8]
    layer_scalar: float     # a bf16 value


FF_TINY = FFConfig("ff_tiny_16tok_h256", TINY, I_dense=192, seed_ff=5)
FF_CANVAS = FFConfig("ff_canvas_256tok_h2816", CANVAS, I_dense=2112, seed_ff=6)
FF_CONFIGS = {c.name: c for c in (FF_TINY, FF_CANVAS)}


def make_ff_weights(cfg: FFConfig) -> FFWeights:
    rng = np.random.default_rng(cfg.seed_ff)
    H, Id = cfg.moe.H, cfg.I_dense
    norms = [to_bf16_bits(rng.uniform(0.8, 1.2, size=H).astype(np.float32)) for _ in range(5)]
    gate = random_qtensor(rng, (Id,), H)
    up = random_qtensor(rng, (Id,), H)
    down = random_qtensor(rng, (H,), Id)
    scalar = float(bf16_bits_as_f32(to_bf16_bits(np.float32(rng.uniform(0.5, 1.5))).reshape(1))[0])
    return FFWeights(*norms, gate, up, down, scalar)

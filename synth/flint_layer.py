"""Seeded synthetic Flint-shaped MoE layers.

Shapes follow the layer the pages describe: hidden size 2048 ("vLLM Day-0
Support for Recursive's Flint", section "Flint Model Architecture"), 256 routed
experts with sigmoid top-6 routing plus one shared expert (same page and
section, "MoE Structure" bullet; also "Flint on Arc Pro B70", section "Setup").
The expert intermediate size is not printed on the pages; 512 is the reading
that makes the stated parameter totals (39.8B total, 2.5B active) come out.

Value distributions (the pages publish no weights):
  router weight  bf16 [E, H]          ~ N(0, 0.02)
  expert w13     bf16 [2*I, H]        ~ N(0, 0.02)   rows [0, I) gate, [I, 2I) up
  expert w2      bf16 [H, I]          ~ N(0, 0.02)
  router bias    fp32 [E]             ~ N(0, 1)      (skewed-load workload only)
  x              bf16 [T, H]          ~ N(0, 1)
  norm gamma     bf16 [H]             ~ 1 + N(0, 0.25)   (pre-norm block only)
  residual r     bf16 [T, H]          ~ s_t * N(0, 1), s_t = 4 exp(N(0, 0.5)) per token,
                                        with 8 outlier channels per layer seed scaled x20

Every tensor has its own random stream, spawned from one integer seed in a
fixed order, so any single tensor can be regenerated without the others:
  child 0            router weight
  child 1, 2         shared expert w13, w2
  child 3+2e, 4+2e   routed expert e w13, w2
  child 3+2E         router bias
  child 4+2E         norm gamma
Activations use a separate SeedSequence keyed by (seed, T, x_seed); the
residual stream another, and its outlier channels one keyed by the seed alone.
The low-latency path's attention side (output projection Wo bf16 [2048, 4096]
~ N(0, 0.02), attention outputs bf16 [T, 4096] ~ N(0, 1), the next layer's
norm gain ~ 1 + N(0, 0.25)) has a domain of its own.

fp32 -> bf16 conversion is round-to-nearest-even on the bit pattern.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

FLINT_HIDDEN = 2048
FLINT_N_EXPERTS = 256
FLINT_TOP_K = 6
FLINT_INTER = 512

WEIGHT_STD = 0.02
X_STD = 1.0
BIAS_STD = 1.0
GAMMA_STD = 0.25
RESID_SCALE = 4.0
RESID_LOG_STD = 0.5
RESID_OUTLIERS = 8
RESID_OUTLIER_GAIN = 20.0

_X_DOMAIN = 0x5EED_0001  # keeps activation streams apart from weight streams
_R_DOMAIN = 0x5EED_0002  # residual-stream inputs of the pre-norm block
_D_DOMAIN = 0x5EED_0003  # dense-MLP weights (layers 0 and 1)
_A_DOMAIN = 0x5EED_0004  # attention side of the low-latency path: Wo, attention outputs, next gain
ATTN_WIDTH = 4096        # attention output width: 32 query heads x head dim 128


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class LayerShape:
    hidden: int = FLINT_HIDDEN
    n_experts: int = FLINT_N_EXPERTS
    top_k: int = FLINT_TOP_K
    inter: int = FLINT_INTER


def _normal_bf16(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seq)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    v *= np.float32(std)
    return f32_to_bf16_bits(v).reshape(shape)


class SyntheticLayer:
    """One seeded MoE layer.  Tensors are generated on first use and cached."""

    def __init__(self, seed: int = 0, shape: LayerShape = LayerShape()):
        self.seed = int(seed)
        self.shape = shape
        E = shape.n_experts
        self._children = np.random.SeedSequence(self.seed).spawn(5 + 2 * E)
        self._cache: dict = {}

    # -- single tensors ---------------------------------------------------
    def router_w(self) -> np.ndarray:
        """bf16 bits [E, H]."""
        key = "router_w"
        if key not in self._cache:
            s = self.shape
            self._cache[key] = _normal_bf16(self._children[0], (s.n_experts, s.hidden), WEIGHT_STD)
        return self._cache[key]

    def router_bias(self) -> np.ndarray:
        """fp32 [E] ~ N(0, 1): the skewed-load workload's per-expert offset."""
        key = "router_b"
        if key not in self._cache:
            E = self.shape.n_experts
            rng = np.random.default_rng(self._children[3 + 2 * E])
            self._cache[key] = (rng.standard_normal(E, dtype=np.float32) * np.float32(BIAS_STD)).astype(np.float32)
        return self._cache[key]

    def norm_weight(self) -> np.ndarray:
        """bf16 bits [H]: the pre-norm block's RMSNorm gain, ~ 1 + N(0, 0.25)."""
        key = "gamma"
        if key not in self._cache:
            rng = np.random.default_rng(self._children[4 + 2 * self.shape.n_experts])
            g = np.float32(1.0) + rng.standard_normal(self.shape.hidden, dtype=np.float32) * np.float32(GAMMA_STD)
            self._cache[key] = f32_to_bf16_bits(g)
        return self._cache[key]

    def _child_w13(self, e: int):
        return self._children[1] if e < 0 else self._children[3 + 2 * e]

    def _child_w2(self, e: int):
        return self._children[2] if e < 0 else self._children[4 + 2 * e]

    def w13(self, e: int) -> np.ndarray:
        """bf16 bits [2I, H] of routed expert e, or of the shared expert if e < 0."""
        s = self.shape
        return _normal_bf16(self._child_w13(e), (2 * s.inter, s.hidden), WEIGHT_STD)

    def w2(self, e: int) -> np.ndarray:
        """bf16 bits [H, I] of routed expert e, or of the shared expert if e < 0."""
        s = self.shape
        return _normal_bf16(self._child_w2(e), (s.hidden, s.inter), WEIGHT_STD)

    # -- whole banks --------------------------------------------------------
    def routed_banks(self, threads: int | None = None):
        """(w13 [E, 2I, H], w2 [E, H, I]) bf16 bits, generated in parallel."""
        if "banks" not in self._cache:
            s = self.shape
            E = s.n_experts
            w13 = np.empty((E, 2 * s.inter, s.hidden), dtype=np.uint16)
            w2 = np.empty((E, s.hidden, s.inter), dtype=np.uint16)

            def fill(e):
                w13[e] = self.w13(e)
                w2[e] = self.w2(e)

            n = threads or min(8, os.cpu_count() or 1)
            with ThreadPoolExecutor(max_workers=n) as ex:
                list(ex.map(fill, range(E)))
            self._cache["banks"] = (w13, w2)
        return self._cache["banks"]

    def shared(self):
        """(w13 [2I, H], w2 [H, I]) bf16 bits of the shared expert."""
        if "shared" not in self._cache:
            self._cache["shared"] = (self.w13(-1), self.w2(-1))
        return self._cache["shared"]

    def expert(self, e: int):
        """(w13, w2) bf16 bits of expert e (shared if e < 0), from the bank when built."""
        if e < 0:
            return self.shared()
        if "banks" in self._cache:
            w13, w2 = self._cache["banks"]
            return w13[e], w2[e]
        return self.w13(e), self.w2(e)


def make_x(T: int, hidden: int = FLINT_HIDDEN, seed: int = 0, x_seed: int = 0) -> np.ndarray:
    """bf16 bits [T, H] ~ N(0, 1), keyed by (seed, T, x_seed)."""
    seq = np.random.SeedSequence([_X_DOMAIN, int(seed), int(T), int(x_seed)])
    return _normal_bf16(seq, (int(T), int(hidden)), X_STD)


def make_residual(T: int, hidden: int = FLINT_HIDDEN, seed: int = 0, x_seed: int = 0) -> np.ndarray:
    """bf16 bits [T, H] of a residual stream, keyed by (seed, T, x_seed).

    Token t is s_t * N(0, 1) with s_t = 4 exp(N(0, 0.5)); the same 8 channels
    (chosen by the seed alone, like a trained model's outlier features) are
    scaled by 20 in every token."""
    ch = np.random.default_rng(np.random.SeedSequence([_R_DOMAIN, int(seed)]))
    outliers = ch.choice(int(hidden), size=RESID_OUTLIERS, replace=False)
    rng = np.random.default_rng(np.random.SeedSequence([_R_DOMAIN, int(seed), int(T), int(x_seed)]))
    s = np.float32(RESID_SCALE) * np.exp(rng.standard_normal((int(T), 1), dtype=np.float32) * np.float32(RESID_LOG_STD))
    v = rng.standard_normal((int(T), int(hidden)), dtype=np.float32) * s
    v[:, outliers] *= np.float32(RESID_OUTLIER_GAIN)
    return f32_to_bf16_bits(v.astype(np.float32)).reshape(int(T), int(hidden))


class SyntheticDenseMLP:
    """Seeded weights of a dense SwiGLU MLP: w13 bf16 [2 I_d, H] (gate rows
    first) and w2 bf16 [H, I_d], both ~ N(0, 0.02), each from its own stream
    keyed by (seed, I_d); the norm gain from a third, ~ 1 + N(0, 0.25)."""

    def __init__(self, seed: int = 0, inter: int = 14336, hidden: int = FLINT_HIDDEN):
        self.seed, self.inter, self.hidden = int(seed), int(inter), int(hidden)
        self._seqs = np.random.SeedSequence([_D_DOMAIN, self.seed, self.inter]).spawn(3)
        self._cache: dict = {}

    def w13(self) -> np.ndarray:
        if "w13" not in self._cache:
            self._cache["w13"] = _normal_bf16(self._seqs[0], (2 * self.inter, self.hidden), WEIGHT_STD)
        return self._cache["w13"]

    def w2(self) -> np.ndarray:
        if "w2" not in self._cache:
            self._cache["w2"] = _normal_bf16(self._seqs[1], (self.hidden, self.inter), WEIGHT_STD)
        return self._cache["w2"]

    def norm_weight(self) -> np.ndarray:
        if "gamma" not in self._cache:
            rng = np.random.default_rng(self._seqs[2])
            g = np.float32(1.0) + rng.standard_normal(self.hidden, dtype=np.float32) * np.float32(GAMMA_STD)
            self._cache["gamma"] = f32_to_bf16_bits(g)
        return self._cache["gamma"]


def make_o_proj(seed: int = 0, hidden: int = FLINT_HIDDEN, width: int = ATTN_WIDTH) -> np.ndarray:
    """bf16 bits [H, 4096] of an attention output projection, ~ N(0, 0.02), keyed by seed."""
    return _normal_bf16(np.random.SeedSequence([_A_DOMAIN, int(seed), 0]), (int(hidden), int(width)),
                        WEIGHT_STD)


def make_attn(T: int, seed: int = 0, x_seed: int = 0, width: int = ATTN_WIDTH) -> np.ndarray:
    """bf16 bits [T, 4096] of attention outputs (per-head weighted sums of
    values), ~ N(0, 1), keyed by (seed, T, x_seed)."""
    seq = np.random.SeedSequence([_A_DOMAIN, int(seed), 1, int(T), int(x_seed)])
    return _normal_bf16(seq, (int(T), int(width)), X_STD)


def make_next_gain(seed: int = 0, hidden: int = FLINT_HIDDEN) -> np.ndarray:
    """bf16 bits [H]: the next layer's RMSNorm gain, ~ 1 + N(0, 0.25), keyed by seed."""
    rng = np.random.default_rng(np.random.SeedSequence([_A_DOMAIN, int(seed), 2]))
    g = np.float32(1.0) + rng.standard_normal(int(hidden), dtype=np.float32) * np.float32(GAMMA_STD)
    return f32_to_bf16_bits(g)

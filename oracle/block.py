"""Plain fp64 oracle of the pre-norm MoE block — test infrastructure only.

Flint is a pre-norm decoder ("vLLM Day-0 Support for Recursive's Flint",
section "Flint Model Architecture", the paragraph before the bullets): the
block input r (the residual stream) is normalised before the feed-forward
layer, and the layer's output is added back to r.  The norm is RMSNorm, whose
kernel divides by the square root of the mean square and writes bf16 ("Flint
on Arc Pro B70", section "norm.py: Triton kernels that assumed CUDA"):

    n   = bf16( r / sqrt(mean_k r[k]^2 + eps) * gamma )
    out = r + MoE(n)

Readings where the pages are silent (each listed with its reason in the design
notes): eps = 1e-6; the normalised activations are rounded once to bf16,
round to nearest even (the norm kernel's output is bf16 and the MoE takes bf16
activations); the MoE output is not rounded before the residual add; the sum
is rounded once to bf16 by whoever stores it (this module returns it in fp64).

The MoE itself is ``oracle.moe.moe_token``; this module adds only the norm,
the bf16 rounding of its output and the residual add.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .moe import OracleLayer, TokenResult, bf16_to_f64, moe_token

DEFAULT_EPS = 1e-6


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in one step; uint16 bits.

    A bf16 value has 8 significant bits.  For |v| in [2^(e-1), 2^e) the bf16
    spacing is 2^(e-8), down to the subnormal spacing 2^-133 (e clamped at
    -125).  v / spacing is exact in fp64, ``np.rint`` rounds it half to even,
    and the rounded multiple of the spacing is exact in fp32, whose top half is
    the bf16 pattern.  Values past the largest bf16 round to infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(v / q) * q
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rmsnorm(r: np.ndarray, gamma: np.ndarray, eps: float = DEFAULT_EPS) -> np.ndarray:
    """r / sqrt(mean(r^2) + eps) * gamma over the last axis, in fp64 (no rounding)."""
    r = np.asarray(r, dtype=np.float64)
    ms = np.mean(r * r, axis=-1, keepdims=True)
    return r / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


@dataclass
class BlockResult:
    out: np.ndarray          # fp64 [H]: r + MoE(n), not yet rounded
    normed_bits: np.ndarray  # uint16 [H]: n, the MoE's bf16 input
    normed_f64: np.ndarray   # fp64 [H]: n before its bf16 rounding
    moe: TokenResult         # the MoE on n (ids, weights, gap, ...)

    # The grading helpers read these names from a token result.
    @property
    def ids(self):
        return self.moe.ids

    @property
    def gap(self):
        return self.moe.gap


def block_token(layer: OracleLayer, r_bits: np.ndarray, gamma_bits: np.ndarray,
                eps: float = DEFAULT_EPS, renormalize: bool = True, routed_scale: float = 1.0,
                expert_cache: Optional[dict] = None) -> BlockResult:
    """The pre-norm block on one token (bf16 bits [H] of r; gamma bf16 bits [H])."""
    r = bf16_to_f64(r_bits).reshape(layer.hidden)
    gamma = bf16_to_f64(gamma_bits).reshape(layer.hidden)
    n64 = rmsnorm(r, gamma, eps)
    n_bits = f64_to_bf16_bits(n64)
    res = moe_token(layer, n_bits, renormalize, routed_scale, expert_cache)
    return BlockResult(out=r + res.out, normed_bits=n_bits, normed_f64=n64, moe=res)


def block_forward(layer: OracleLayer, r_bits: np.ndarray, gamma_bits: np.ndarray,
                  eps: float = DEFAULT_EPS, renormalize: bool = True, routed_scale: float = 1.0,
                  tokens=None):
    """Per-token loop over r bits [T, H] (or the listed token indices)."""
    R = np.asarray(r_bits, dtype=np.uint16).reshape(-1, layer.hidden)
    idx = range(R.shape[0]) if tokens is None else tokens
    cache: dict = {}
    return [block_token(layer, R[t], gamma_bits, eps, renormalize, routed_scale, cache) for t in idx]

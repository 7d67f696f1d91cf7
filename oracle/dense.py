"""Plain fp64 oracle of Flint's dense MLP (layers 0 and 1) — test infrastructure only.

The first two layers of Flint use a dense MLP instead of the MoE ("vLLM Day-0
Support for Recursive's Flint", section "Flint Model Architecture", bullet
"MoE Structure").  Its form is read as the experts' SwiGLU ("Flint on Arc Pro
B70", section "norm.py: Triton kernels that assumed CUDA": SiLU of the gate
projection times the up projection), with one intermediate size I_d that the
pages do not print; the weights are w13 = [gate rows; up rows] [2 I_d, H] and
w2 [H, I_d], as for an expert:

    h   = silu(W13[0:I_d] x) * (W13[I_d:2 I_d] x)
    out = W2 h

and, as a pre-norm block like every Flint layer (same page and section, the
paragraph before the bullets), out = r + MLP(bf16(RMSNorm(r) * gamma)).
fp64 throughout; the GEMV step is numpy's ``@``.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .block import DEFAULT_EPS, f64_to_bf16_bits, rmsnorm
from .moe import bf16_to_f64, silu


@dataclass
class DenseMLP:
    """Weights as bf16 bit patterns: w13 [2 I_d, H] (gate rows first), w2 [H, I_d]."""
    hidden: int
    inter: int
    w13_bits: np.ndarray
    w2_bits: np.ndarray

    def f64(self):
        w13 = bf16_to_f64(self.w13_bits).reshape(2 * self.inter, self.hidden)
        w2 = bf16_to_f64(self.w2_bits).reshape(self.hidden, self.inter)
        return w13, w2


def mlp_token(w13: np.ndarray, w2: np.ndarray, x: np.ndarray, inter: int):
    """(out [H], h [I_d]) of one token x [H] (fp64)."""
    g = w13[:inter] @ x
    u = w13[inter:] @ x
    h = silu(g) * u
    return w2 @ h, h


def mlp_forward(mlp: DenseMLP, x_bits: np.ndarray, tokens=None):
    """Per-token loop over x bits [T, H]: list of (out fp64 [H], h fp64 [I_d])."""
    X = np.asarray(x_bits, dtype=np.uint16).reshape(-1, mlp.hidden)
    w13, w2 = mlp.f64()
    idx = range(X.shape[0]) if tokens is None else tokens
    return [mlp_token(w13, w2, bf16_to_f64(X[t]), mlp.inter) for t in idx]


@dataclass
class DenseBlockResult:
    out: np.ndarray          # fp64 [H]: r + MLP(n)
    mlp_out: np.ndarray      # fp64 [H]: MLP(n)
    normed_bits: np.ndarray  # uint16 [H]
    normed_f64: np.ndarray   # fp64 [H], before rounding
    h: np.ndarray            # fp64 [I_d]


def mlp_block_forward(mlp: DenseMLP, r_bits: np.ndarray, gamma_bits: np.ndarray,
                      eps: float = DEFAULT_EPS, tokens=None):
    """The pre-norm dense block per token: out = r + MLP(bf16(RMSNorm(r) * gamma))."""
    R = np.asarray(r_bits, dtype=np.uint16).reshape(-1, mlp.hidden)
    gamma = bf16_to_f64(gamma_bits).reshape(mlp.hidden)
    w13, w2 = mlp.f64()
    idx = range(R.shape[0]) if tokens is None else tokens
    res = []
    for t in idx:
        r = bf16_to_f64(R[t])
        n64 = rmsnorm(r, gamma, eps)
        nb = f64_to_bf16_bits(n64)
        y, h = mlp_token(w13, w2, bf16_to_f64(nb), mlp.inter)
        res.append(DenseBlockResult(out=r + y, mlp_out=y, normed_bits=nb, normed_f64=n64, h=h))
    return res

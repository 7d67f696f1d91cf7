"""Expert-grouped fp64 evaluation of the layer for large batches — test infrastructure only.

The same arithmetic as ``oracle.moe.moe_token`` (and ``oracle.block`` /
``oracle.dense``), reorganised so that a whole prefill-sized batch (8192
tokens, "RecursiveSI/flint — vLLM serving recipe", section "Benchmarking",
prefill 8K) can be evaluated in seconds instead of hours:

* the router GEMV of every token is one matrix product X Wr^T;
* sigmoid, top-k (ties to the lower expert index) and the routing weights
  are the per-token definitions applied row-wise;
* each expert's SwiGLU runs once over the tokens routed to it: gather their
  rows, two matrix products for gate and up, SiLU times up, one matrix
  product for down; the weighted result is added to those tokens' rows.

Nothing is blocked, fused or approximated beyond that regrouping: each
token's output is the same sum of the same fp64 terms as the per-token
oracle.  Only the order in which a token's k routed terms are added can
differ (expert order here, rank order there), which moves the fp64 result
by a few units in its last place (~1e-16 relative).
``tests/test_oracle_grouped.py`` pins this module against the per-token
oracle on a full-size layer, token by token.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .block import DEFAULT_EPS, f64_to_bf16_bits, rmsnorm
from .moe import OracleLayer, bf16_to_f64, silu, sigmoid


@dataclass
class GroupedResult:
    out: np.ndarray        # fp64 [T, H]: the layer output (the block: r + layer)
    ids: np.ndarray        # int32 [T, k]: selected experts in rank order
    weights: np.ndarray    # fp64 [T, k]: routing weights
    gaps: np.ndarray       # fp64 [T]: s_(k) - s_(k+1)
    logits: np.ndarray     # fp64 [T, E]
    layer_out: Optional[np.ndarray] = None     # block only: the layer part, fp64 [T, H]
    normed_bits: Optional[np.ndarray] = None   # block only: n, uint16 [T, H]
    normed_f64: Optional[np.ndarray] = None    # block only: n before rounding, fp64 [T, H]


def route_rows(layer: OracleLayer, X: np.ndarray, renormalize: bool = True,
               routed_scale: float = 1.0):
    """Router, sigmoid, top-k and weights for the rows of X (fp64 [T, H]).

    Returns (ids int32 [T, k], weights fp64 [T, k], gaps fp64 [T], logits fp64 [T, E]).
    The ranking sorts the negated scores stably, so equal scores keep their
    ascending expert order: ties go to the lower index, as in ``select_topk``.
    """
    k, E = layer.top_k, layer.n_experts
    Z = X @ layer.router_f64().T
    b = layer.bias_f64()
    if b is not None:
        Z = Z + b[None, :]
    S = sigmoid(Z)
    order = np.argsort(-S, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    rows = np.arange(X.shape[0])
    if k < E:
        gaps = S[rows, order[:, k - 1]] - S[rows, order[:, k]]
    else:
        gaps = np.full(X.shape[0], np.inf)
    sel = np.take_along_axis(S, ids.astype(np.int64), axis=1)
    w = sel / np.sum(sel, axis=1, keepdims=True) if renormalize else sel.copy()
    return ids, w * float(routed_scale), gaps, Z


def _expert_rows(w13: np.ndarray, w2: np.ndarray, Xe: np.ndarray, inter: int) -> np.ndarray:
    """SwiGLU of one expert over the rows of Xe (fp64 [n, H]): y [n, H]."""
    G = Xe @ w13[:inter].T
    U = Xe @ w13[inter:].T
    return (silu(G) * U) @ w2.T


def layer_rows(layer: OracleLayer, X: np.ndarray, renormalize: bool = True,
               routed_scale: float = 1.0):
    """The layer on the rows of X (fp64 [T, H]), grouped by expert.

    Returns (out fp64 [T, H], ids, weights, gaps, logits)."""
    ids, w, gaps, Z = route_rows(layer, X, renormalize, routed_scale)
    sw13, sw2 = layer.expert_f64(-1)
    out = _expert_rows(sw13, sw2, X, layer.inter)
    for e in np.unique(ids):
        tok, rank = np.nonzero(ids == e)          # each token selects e at most once
        w13, w2 = layer.expert_f64(int(e))
        out[tok] += w[tok, rank][:, None] * _expert_rows(w13, w2, X[tok], layer.inter)
    return out, ids, w, gaps, Z


def moe_forward_grouped(layer: OracleLayer, x_bits: np.ndarray, renormalize: bool = True,
                        routed_scale: float = 1.0) -> GroupedResult:
    """The layer on every token of x bits [T, H], evaluated per expert."""
    X = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16)).reshape(-1, layer.hidden)
    out, ids, w, gaps, Z = layer_rows(layer, X, renormalize, routed_scale)
    return GroupedResult(out=out, ids=ids, weights=w, gaps=gaps, logits=Z)


def block_forward_grouped(layer: OracleLayer, r_bits: np.ndarray, gamma_bits: np.ndarray,
                          eps: float = DEFAULT_EPS, renormalize: bool = True,
                          routed_scale: float = 1.0) -> GroupedResult:
    """The pre-norm block (``oracle.block``) on every token of r bits [T, H]:
    n = bf16(RMSNorm(r) * gamma) row by row, the grouped layer on n, plus r."""
    R = bf16_to_f64(np.asarray(r_bits, dtype=np.uint16)).reshape(-1, layer.hidden)
    gamma = bf16_to_f64(gamma_bits).reshape(layer.hidden)
    n64 = rmsnorm(R, gamma, eps)
    nb = f64_to_bf16_bits(n64)
    y, ids, w, gaps, Z = layer_rows(layer, bf16_to_f64(nb).reshape(R.shape), renormalize,
                                    routed_scale)
    return GroupedResult(out=R + y, ids=ids, weights=w, gaps=gaps, logits=Z, layer_out=y,
                         normed_bits=nb, normed_f64=n64)


def mlp_forward_batched(w13_bits: np.ndarray, w2_bits: np.ndarray, x_bits: np.ndarray,
                        hidden: int, inter: int, gamma_bits: Optional[np.ndarray] = None,
                        eps: float = DEFAULT_EPS, chunk: int = 1024):
    """The dense MLP (``oracle.dense``) on every token at once, as matrix
    products over chunks of ``chunk`` tokens (to bound memory).

    Without gamma: returns out fp64 [T, H] = MLP(x).  With gamma (the pre-norm
    block): returns (r + MLP(n), MLP(n)) with n = bf16(RMSNorm(r) * gamma)."""
    w13 = bf16_to_f64(w13_bits).reshape(2 * inter, hidden)
    w2 = bf16_to_f64(w2_bits).reshape(hidden, inter)
    X = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16)).reshape(-1, hidden)
    if gamma_bits is not None:
        gamma = bf16_to_f64(gamma_bits).reshape(hidden)
        A = bf16_to_f64(f64_to_bf16_bits(rmsnorm(X, gamma, eps))).reshape(X.shape)
    else:
        A = X
    y = np.empty_like(X)
    for t0 in range(0, X.shape[0], chunk):
        y[t0:t0 + chunk] = _expert_rows(w13, w2, A[t0:t0 + chunk], inter)
    return y if gamma_bits is None else (X + y, y)

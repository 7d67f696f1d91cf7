"""Plain fp64 oracle of the Flint MoE feed-forward layer — test infrastructure only.

What the layer computes, per token t, as the pages define it:

* 256 routed experts, sigmoid scoring, top-6 selection, plus one always-on
  shared expert ("vLLM Day-0 Support for Recursive's Flint", section "Flint
  Model Architecture", bullet "MoE Structure"; "Flint on Arc Pro B70",
  section "Setup"; "RecursiveSI/flint — vLLM serving recipe", section
  "Guide / Overview").  Hidden size 2048 (Day-0 page, same section).
* The router and expert projections are GEMVs over the token's hidden vector,
  and only the selected experts' weights take part (Day-0 page, section
  "Optimization Strategies", bullet "Small-batch MoE Kernels").
* Each expert is SwiGLU: SiLU of the gate projection times the up projection,
  then the down projection.  The SiLU form is g / (1 + exp(-g)) ("Flint on Arc
  Pro B70", section "norm.py: Triton kernels that assumed CUDA").
* The routed outputs are combined by their routing weights and added to the
  shared expert's output (Day-0 page, section "Optimization Strategies",
  bullet "Low-Latency Decode Path": "expert combine").

Readings where the pages are silent (each listed with its reason in the design
notes): intermediate size 512; shared expert of the same shape, ungated, weight
1; optional router bias added to the logit before the sigmoid; routing weights
renormalised over the selected experts (flag, default on) and multiplied by
``routed_scale`` (default 1); w13 rows [0, I) are gate and [I, 2I) are up;
ranking on the score, ties to the lower expert index; no rounding anywhere
(inputs are exact bf16 / NVFP4, everything else fp64).

All arithmetic is fp64.  Matrix-vector products use numpy's ``@`` as the GEMV
step; everything else is written out per token, with no blocking or fusion.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

from .nvfp4 import nvfp4_dequant


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64.  Exact: bf16 is the top half of fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def router_logits(x: np.ndarray, router_w: np.ndarray, router_b: Optional[np.ndarray]) -> np.ndarray:
    """z_e = sum_k W_r[e, k] x[k] (+ b_e): the router GEMV over all experts.

    x fp64 [H]; router_w fp64 [E, H]; router_b fp64 [E] or None.
    """
    z = router_w @ x
    if router_b is not None:
        z = z + router_b
    return z


def sigmoid(z: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-z)), the sigmoid scoring of the MoE Structure bullet."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU in the form the B70 write-up prints: g / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def select_topk(scores: np.ndarray, k: int):
    """The k experts with the largest scores, ties to the lower index.

    Returns (ids int32 [k] in rank order, gap) where gap = s_(k) - s_(k+1) is
    the score distance between the last selected and the first unselected
    expert (inf when k equals the number of experts).
    """
    s = np.asarray(scores, dtype=np.float64)
    E = s.shape[0]
    order = sorted(range(E), key=lambda e: (-s[e], e))
    ids = np.array(order[:k], dtype=np.int32)
    gap = float(s[order[k - 1]] - s[order[k]]) if k < E else float("inf")
    return ids, gap


def routing_weights(scores: np.ndarray, ids: np.ndarray, renormalize: bool = True,
                    routed_scale: float = 1.0) -> np.ndarray:
    """w_j = s_{ids_j} / sum_i s_{ids_i} (if renormalize) times routed_scale."""
    sel = np.asarray(scores, dtype=np.float64)[np.asarray(ids)]
    w = sel / np.sum(sel) if renormalize else sel.copy()
    return w * float(routed_scale)


def expert_forward(w13: np.ndarray, w2: np.ndarray, x: np.ndarray, inter: int):
    """One SwiGLU expert on one token.

    w13 fp64 [2I, H] (rows [0, I) gate, [I, 2I) up); w2 fp64 [H, I]; x fp64 [H].
    g = W_gate x, u = W_up x, h = silu(g) * u, y = W2 h.  Returns (y [H], h [I]).
    """
    g = w13[:inter] @ x
    u = w13[inter:] @ x
    h = silu(g) * u
    return w2 @ h, h


@dataclass
class OracleLayer:
    """The layer's parameters as the oracle reads them.

    ``expert_raw(e)`` returns expert e's stored weights (e < 0: the shared
    expert): for ``fmt == "bf16"`` a pair (w13 bits [2I, H], w2 bits [H, I]);
    for ``fmt == "nvfp4"`` a pair of (packed, scales, gscale) triples.
    """

    hidden: int
    n_experts: int
    top_k: int
    inter: int
    router_w_bits: np.ndarray
    router_b: Optional[np.ndarray]
    expert_raw: Callable[[int], tuple]
    fmt: str = "bf16"
    _router_f64: Optional[np.ndarray] = field(default=None, repr=False)

    def router_f64(self) -> np.ndarray:
        if self._router_f64 is None:
            self._router_f64 = bf16_to_f64(self.router_w_bits).reshape(self.n_experts, self.hidden)
        return self._router_f64

    def bias_f64(self) -> Optional[np.ndarray]:
        if self.router_b is None:
            return None
        return np.asarray(self.router_b, dtype=np.float32).astype(np.float64)

    def expert_f64(self, e: int):
        """(w13 fp64 [2I, H], w2 fp64 [H, I]) of expert e (shared if e < 0)."""
        a, b = self.expert_raw(e)
        if self.fmt == "bf16":
            w13 = bf16_to_f64(a).reshape(2 * self.inter, self.hidden)
            w2 = bf16_to_f64(b).reshape(self.hidden, self.inter)
        elif self.fmt == "nvfp4":
            w13 = nvfp4_dequant(*a).reshape(2 * self.inter, self.hidden)
            w2 = nvfp4_dequant(*b).reshape(self.hidden, self.inter)
        else:
            raise ValueError(f"unknown weight format {self.fmt!r}")
        return w13, w2


@dataclass
class TokenResult:
    out: np.ndarray          # fp64 [H]
    ids: np.ndarray          # int32 [k], rank order
    weights: np.ndarray      # fp64 [k]
    gap: float               # s_(k) - s_(k+1)
    logits: np.ndarray       # fp64 [E]
    scores: np.ndarray       # fp64 [E]
    h_routed: np.ndarray     # fp64 [k, I]
    h_shared: np.ndarray     # fp64 [I]


def moe_token(layer: OracleLayer, x_bits: np.ndarray, renormalize: bool = True,
              routed_scale: float = 1.0, expert_cache: Optional[dict] = None) -> TokenResult:
    """The whole layer on one token (bf16 bits [H]), in the pages' order:
    router GEMV -> sigmoid -> top-k -> routing weights -> SwiGLU experts
    (selected + shared) -> combine."""
    cache = {} if expert_cache is None else expert_cache

    def weights_of(e):
        if e not in cache:
            cache[e] = layer.expert_f64(e)
        return cache[e]

    x = bf16_to_f64(x_bits).reshape(layer.hidden)
    z = router_logits(x, layer.router_f64(), layer.bias_f64())
    s = sigmoid(z)
    ids, gap = select_topk(s, layer.top_k)
    w = routing_weights(s, ids, renormalize, routed_scale)

    w13, w2 = weights_of(-1)
    y_shared, h_shared = expert_forward(w13, w2, x, layer.inter)
    out = y_shared.copy()
    h_routed = np.empty((layer.top_k, layer.inter), dtype=np.float64)
    for j, e in enumerate(ids):
        w13, w2 = weights_of(int(e))
        y, h = expert_forward(w13, w2, x, layer.inter)
        h_routed[j] = h
        out = out + w[j] * y
    return TokenResult(out=out, ids=ids, weights=w, gap=gap, logits=z, scores=s,
                       h_routed=h_routed, h_shared=h_shared)


def moe_forward(layer: OracleLayer, x_bits: np.ndarray, renormalize: bool = True,
                routed_scale: float = 1.0, tokens=None):
    """Per-token loop over x bits [T, H] (or the listed token indices)."""
    X = np.asarray(x_bits, dtype=np.uint16).reshape(-1, layer.hidden)
    idx = range(X.shape[0]) if tokens is None else tokens
    cache: dict = {}
    return [moe_token(layer, X[t], renormalize, routed_scale, cache) for t in idx]


def route_all(layer: OracleLayer, x_bits: np.ndarray, renormalize: bool = True,
              routed_scale: float = 1.0):
    """Router, sigmoid, top-k and weights for every token (no experts).

    Returns (ids int32 [T, k], weights fp64 [T, k], gaps fp64 [T], logits fp64 [T, E]).
    """
    X = np.asarray(x_bits, dtype=np.uint16).reshape(-1, layer.hidden)
    T = X.shape[0]
    ids = np.empty((T, layer.top_k), dtype=np.int32)
    w = np.empty((T, layer.top_k), dtype=np.float64)
    gaps = np.empty(T, dtype=np.float64)
    logits = np.empty((T, layer.n_experts), dtype=np.float64)
    Wr, b = layer.router_f64(), layer.bias_f64()
    for t in range(T):
        z = router_logits(bf16_to_f64(X[t]), Wr, b)
        s = sigmoid(z)
        ids[t], gaps[t] = select_topk(s, layer.top_k)
        w[t] = routing_weights(s, ids[t], renormalize, routed_scale)
        logits[t] = z
    return ids, w, gaps, logits


def bucket(ids: np.ndarray, n_experts: int) -> dict:
    """Token -> expert bucketing of the selected (token, rank) slots.

    A slot is s = t * k + j for token t and rank j.  Returns
      counts  int32 [E]     slots routed to each expert
      offsets int32 [E + 1] exclusive prefix sum of counts
      active  int32 [n]     experts with count > 0, ascending (the union U)
      slots   int32 [T*k]   slot ids grouped by expert (ascending expert),
                            ascending slot id within an expert
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int32)
    lists = [[] for _ in range(n_experts)]
    for s, e in enumerate(flat):
        counts[e] += 1
        lists[e].append(s)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    active = np.array([e for e in range(n_experts) if counts[e] > 0], dtype=np.int32)
    slots = np.array([s for e in range(n_experts) for s in lists[e]], dtype=np.int32)
    return {"counts": counts, "offsets": offsets, "active": active, "slots": slots}

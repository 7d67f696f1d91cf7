"""Plain fp64 oracle of the low-latency decode path around the MoE layer — test
infrastructure only.

"vLLM Day-0 Support for Recursive's Flint", section "Optimization
Strategies", bullet "Low-Latency Decode Path": for batches of up to 8
requests the MoE layer's routing and expert combine are fused into the
neighbouring GEMV kernels.  The neighbours of the MoE layer in a pre-norm
decoder ("Flint Model Architecture": 49 pre-norm layers, hidden size 2048;
GQA with 32 query heads) are, before it, the attention's output projection
and the residual add with the post-attention RMSNorm, and after it, the
residual add and the next layer's input RMSNorm.  Per token:

    r1  = bf16( r + Wo a )                       attention output a [4096], Wo [2048, 4096]
    n   = bf16( RMSNorm(r1) * gamma )            the MoE's pre-norm (oracle.block)
    r2  = bf16( r1 + MoE(n) )                    the residual stream leaving the layer
    n2  = bf16( RMSNorm(r2) * gamma_next )       the next layer's normalised input

Readings where the pages are silent (each listed with its reason in the
design notes): the attention output is 32 heads x 128 = 4096 wide; the
residual stream is bf16 and each residual add is rounded once (to nearest
even); both norms use the form and eps of ``oracle.block``.  The MoE itself
is ``oracle.moe.moe_token`` via ``oracle.block.block_token``.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .block import DEFAULT_EPS, BlockResult, block_token, f64_to_bf16_bits, rmsnorm
from .moe import OracleLayer, bf16_to_f64

ATTN_WIDTH = 4096     # 32 query heads x head dim 128


@dataclass
class DecoderResult:
    r1_f64: np.ndarray        # fp64 [H]: r + Wo a before its rounding
    r1_bits: np.ndarray       # uint16 [H]
    block: BlockResult        # the pre-norm MoE block on r1 (n, ids, weights, gap, r1 + MoE)
    r2_bits: np.ndarray       # uint16 [H]: bf16(r1 + MoE(n))
    n2_f64: Optional[np.ndarray]   # fp64 [H]: RMSNorm(r2) * gamma_next before rounding
    n2_bits: Optional[np.ndarray]  # uint16 [H]

    # The grading helpers read these names from a token result.
    @property
    def ids(self):
        return self.block.ids

    @property
    def gap(self):
        return self.block.gap

    @property
    def out(self):
        """r1 + MoE(n), unrounded (what r2 rounds)."""
        return self.block.out

    @property
    def moe(self):
        return self.block.moe


def o_proj(wo_f64: np.ndarray, attn_bits: np.ndarray) -> np.ndarray:
    """Wo a: the attention output projection of one token (GEMV, fp64)."""
    return wo_f64 @ bf16_to_f64(attn_bits).reshape(wo_f64.shape[1])


def decoder_token(layer: OracleLayer, wo_f64: np.ndarray, attn_bits: np.ndarray, r_bits: np.ndarray,
                  gamma_bits: np.ndarray, gamma_next_bits: Optional[np.ndarray] = None,
                  eps: float = DEFAULT_EPS, renormalize: bool = True, routed_scale: float = 1.0,
                  expert_cache: Optional[dict] = None) -> DecoderResult:
    """The path on one token: attention output bits [4096], residual bits [H]."""
    r = bf16_to_f64(r_bits).reshape(layer.hidden)
    r1 = r + o_proj(wo_f64, attn_bits)
    r1_bits = f64_to_bf16_bits(r1)
    blk = block_token(layer, r1_bits, gamma_bits, eps, renormalize, routed_scale, expert_cache)
    r2_bits = f64_to_bf16_bits(blk.out)
    n2_f64 = n2_bits = None
    if gamma_next_bits is not None:
        n2_f64 = rmsnorm(bf16_to_f64(r2_bits), bf16_to_f64(gamma_next_bits), eps)
        n2_bits = f64_to_bf16_bits(n2_f64)
    return DecoderResult(r1_f64=r1, r1_bits=r1_bits, block=blk, r2_bits=r2_bits, n2_f64=n2_f64,
                         n2_bits=n2_bits)


def decoder_forward(layer: OracleLayer, wo_bits: np.ndarray, attn_bits: np.ndarray,
                    r_bits: np.ndarray, gamma_bits: np.ndarray,
                    gamma_next_bits: Optional[np.ndarray] = None, eps: float = DEFAULT_EPS,
                    renormalize: bool = True, routed_scale: float = 1.0):
    """Per-token loop over attn bits [T, W] and r bits [T, H]; Wo bits [H, W]
    (W = 4096 for Flint)."""
    wo_bits = np.asarray(wo_bits, dtype=np.uint16)
    width = wo_bits.shape[1] if wo_bits.ndim == 2 else ATTN_WIDTH
    A = np.asarray(attn_bits, dtype=np.uint16).reshape(-1, width)
    R = np.asarray(r_bits, dtype=np.uint16).reshape(-1, layer.hidden)
    wo = bf16_to_f64(wo_bits).reshape(layer.hidden, width)
    cache: dict = {}
    return [decoder_token(layer, wo, A[t], R[t], gamma_bits, gamma_next_bits, eps, renormalize,
                          routed_scale, cache) for t in range(A.shape[0])]

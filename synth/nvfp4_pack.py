"""NVFP4 byte encoding of synthetic bf16 weights (input preparation only).

The pages name the format (an NVFP4 checkpoint served weight-only as W4A16
with bf16 activations: "vLLM Day-0 Support for Recursive's Flint", section
"Flint Model Overview and Capabilities"; "RecursiveSI/flint — vLLM serving
recipe", section "Guide / Overview") but print neither its byte layout nor the
quantiser.  This encoder is the reading used throughout this repository:

  * elements: FP4 E2M1 codes, two per byte, the even K index in the low nibble;
    nibble bit 3 is the sign, bits 2..0 index the magnitudes
    {0, 0.5, 1, 1.5, 2, 3, 4, 6};
  * one FP8 E4M3FN scale byte per 16 consecutive K elements, row-major
    [rows][K/16];
  * one fp32 scale per tensor;  W ~= e2m1(q) * e4m3(s_block) * g_tensor.

Quantiser: g = amax|W| / (6 * 448); s_block = e4m3(amax_block / (6 g)),
rounded to nearest-even and saturated at 448; q = e2m1(W / (s_block g)),
rounded to nearest-even, clamped to +-6; q = 0 where s_block is 0.
It only makes inputs: parity is graded against the oracle evaluated on the
decoded bytes, so nothing downstream depends on these rounding choices.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .flint_layer import bf16_bits_to_f32

E2M1_MAX = 6.0
E4M3_MAX = 448.0
BLOCK = 16

_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_E2M1_MIDS = (_E2M1_MAGS[:-1] + _E2M1_MAGS[1:]) / 2.0


@dataclass
class NvFp4Tensor:
    packed: np.ndarray   # uint8 [rows, K/2]
    scales: np.ndarray   # uint8 [rows, K/16]  (E4M3FN bytes)
    gscale: np.float32   # per-tensor fp32 scale


def _e2m1_code(a: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code (ties to the even code) for a >= 0."""
    up = np.searchsorted(_E2M1_MIDS, a, side="right")
    tie = (up > 0) & (a == _E2M1_MIDS[np.maximum(up - 1, 0)])
    return np.where(tie & (up % 2 == 1), up - 1, up).astype(np.uint8)


def _e4m3_bytes(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.minimum(v, E4M3_MAX).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _e4m3_values(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def quantize_nvfp4(w_bf16_bits: np.ndarray) -> NvFp4Tensor:
    """Encode one bf16 weight matrix [rows, K] (K a multiple of 16) as NVFP4."""
    w = bf16_bits_to_f32(w_bf16_bits).astype(np.float64)
    rows, K = w.shape
    assert K % BLOCK == 0
    amax = float(np.max(np.abs(w)))
    g = np.float32(amax / (E2M1_MAX * E4M3_MAX)) if amax > 0 else np.float32(1.0)
    gd = float(g)
    blocks = w.reshape(rows, K // BLOCK, BLOCK)
    bmax = np.max(np.abs(blocks), axis=2)
    s_bytes = _e4m3_bytes(bmax / (E2M1_MAX * gd))
    s_vals = _e4m3_values(s_bytes)
    denom = s_vals[:, :, None] * gd
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(denom > 0, blocks / denom, 0.0)
    r = np.clip(r, -E2M1_MAX, E2M1_MAX)
    code = _e2m1_code(np.abs(r))
    neg = (r < 0) & (code != 0)
    nib = (code | (neg.astype(np.uint8) << 3)).reshape(rows, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return NvFp4Tensor(packed=np.ascontiguousarray(packed),
                       scales=np.ascontiguousarray(s_bytes.astype(np.uint8)),
                       gscale=g)

"""Grading of a layer output against the oracle — test infrastructure only.

Rules: a token whose oracle gap between the k-th and (k+1)-th sigmoid score is
below ``gap_min`` (1e-5) is reported and excluded from both checks.  For the
others, the selected index *sets* must be equal, and
max |out - oracle| <= tol * RMS(oracle out) over those tokens and all columns
(tol = 2e-2 for bf16 weights, 5e-2 for NVFP4).

The pre-norm block (``grade_block``) adds the residual r before the one bf16
rounding of the output, so |r| can dwarf the layer's part: there the bound is
tol * RMS(oracle layer output) + 2^-8 |oracle out| per element, the second term
being the bf16 rounding of the stored sum (half a bf16 spacing is at most
2^-8 of the value).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .moe import bf16_to_f64

GAP_MIN = 1e-5
TOL_BF16 = 2e-2
TOL_NVFP4 = 5e-2


@dataclass
class Grade:
    n_tokens: int
    excluded: list
    id_mismatch: list
    max_err: float
    rms: float
    ratio: float       # max_err / rms
    tol: float

    @property
    def ok(self) -> bool:
        return not self.id_mismatch and self.ratio <= self.tol

    def __str__(self):
        return (f"tokens={self.n_tokens} excluded={len(self.excluded)} "
                f"id_mismatch={self.id_mismatch[:8]} max_err={self.max_err:.3e} "
                f"rms={self.rms:.4f} ratio={self.ratio:.4f} tol={self.tol}")


def grade(out_bits: np.ndarray, ids: np.ndarray, results, tokens=None, tol: float = TOL_BF16,
          gap_min: float = GAP_MIN) -> Grade:
    """out_bits: bf16 bits [T, H] from the device; ids: int [T, k]; results:
    oracle TokenResults for ``tokens`` (default: every row, in order)."""
    tokens = list(range(len(results))) if tokens is None else list(tokens)
    out = bf16_to_f64(np.asarray(out_bits)).reshape(np.asarray(out_bits).shape)
    excluded, mism, keep = [], [], []
    for t, r in zip(tokens, results):
        if r.gap < gap_min:
            excluded.append(t)
            continue
        if set(np.asarray(ids[t]).tolist()) != set(r.ids.tolist()):
            mism.append(t)
        keep.append((t, r))
    if not keep:
        return Grade(len(tokens), excluded, mism, 0.0, 0.0, 0.0, tol)
    ref = np.stack([r.out for _, r in keep])
    got = np.stack([out[t] for t, _ in keep])
    err = float(np.max(np.abs(got - ref)))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return Grade(len(tokens), excluded, mism, err, rms, err / rms if rms > 0 else float("inf"), tol)


def grade_block(out_bits: np.ndarray, ids: np.ndarray, results, tokens=None, tol: float = TOL_BF16,
                gap_min: float = GAP_MIN) -> Grade:
    """Like ``grade`` for BlockResults: ``max_err`` is the largest excess of
    |out - oracle| over the rounding allowance 2^-8 |oracle|, ``rms`` the RMS
    of the oracle's layer part (out - r)."""
    tokens = list(range(len(results))) if tokens is None else list(tokens)
    out = bf16_to_f64(np.asarray(out_bits)).reshape(np.asarray(out_bits).shape)
    excluded, mism, keep = [], [], []
    for t, r in zip(tokens, results):
        if r.gap < gap_min:
            excluded.append(t)
            continue
        if set(np.asarray(ids[t]).tolist()) != set(r.ids.tolist()):
            mism.append(t)
        keep.append((t, r))
    if not keep:
        return Grade(len(tokens), excluded, mism, 0.0, 0.0, 0.0, tol)
    ref = np.stack([r.out for _, r in keep])
    moe = np.stack([r.moe.out for _, r in keep])
    got = np.stack([out[t] for t, _ in keep])
    excess = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)
    err = float(max(0.0, np.max(excess)))
    rms = float(np.sqrt(np.mean(moe ** 2)))
    return Grade(len(tokens), excluded, mism, err, rms, err / rms if rms > 0 else float("inf"), tol)

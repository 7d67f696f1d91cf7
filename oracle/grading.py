"""Grading of a layer output against the oracle — test infrastructure only.

Rules: a token whose oracle gap between the k-th and (k+1)-th sigmoid score is
below ``gap_min`` (1e-5) is reported and excluded from both checks.  For the
others, the selected index *sets* must be equal, and
max |out - oracle| <= tol * RMS(oracle out) over those tokens and all columns
(tol = 2e-2 for bf16 weights, 5e-2 for NVFP4).  A grade over no token at all
(every token excluded, or none given) fails: it has checked nothing.

The pre-norm block (``grade_block``) adds the residual r before the one bf16
rounding of the output, so |r| can dwarf the layer's part: there the bound is
tol * RMS(oracle layer output) + 2^-8 |oracle out| per element, the second term
being the bf16 rounding of the stored sum (half a bf16 spacing is at most
2^-8 of the value).

``grade`` / ``grade_block`` take per-token oracle results (``moe_forward``,
``block_forward``); ``grade_arrays`` / ``grade_block_arrays`` take the
whole-batch arrays of ``oracle.grouped``.  Both forms share one core.
``tests/test_grading.py`` pins the checker on planted errors of known size.
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
    n_graded: int = 0  # tokens that took part in the output check
    worst_token: int = -1

    @property
    def ok(self) -> bool:
        return self.n_graded > 0 and not self.id_mismatch and self.ratio <= self.tol

    def __str__(self):
        return (f"tokens={self.n_tokens} graded={self.n_graded} excluded={len(self.excluded)} "
                f"id_mismatch={self.id_mismatch[:8]} max_err={self.max_err:.3e} "
                f"rms={self.rms:.4f} ratio={self.ratio:.4f} tol={self.tol} "
                f"worst_token={self.worst_token}")


def _core(got: np.ndarray, ref: np.ndarray, scale_ref: np.ndarray, ids: np.ndarray,
          ref_ids: np.ndarray, gaps: np.ndarray, tokens: np.ndarray, tol: float, gap_min: float,
          rounding_allowance: bool) -> Grade:
    """got, ref, scale_ref: fp64 [n, H]; ids, ref_ids: [n, k]; gaps [n];
    tokens: the token index of each row (for reporting)."""
    n = got.shape[0]
    keep = np.asarray(gaps, dtype=np.float64) >= gap_min
    excluded = [int(t) for t in tokens[~keep]]
    a = np.sort(np.asarray(ids, dtype=np.int64), axis=1)
    b = np.sort(np.asarray(ref_ids, dtype=np.int64), axis=1)
    mism_rows = keep & np.any(a != b, axis=1)
    mism = [int(t) for t in tokens[mism_rows]]
    if not keep.any():
        return Grade(n, excluded, mism, 0.0, 0.0, float("inf"), tol, 0, -1)
    g, r, s = got[keep], ref[keep], scale_ref[keep]
    if rounding_allowance:
        excess = np.abs(g - r) - 2.0 ** -8 * np.abs(r)
        per_tok = np.maximum(0.0, np.max(excess, axis=1))
    else:
        per_tok = np.max(np.abs(g - r), axis=1)
    worst = int(np.argmax(per_tok))
    err = float(per_tok[worst])
    rms = float(np.sqrt(np.mean(s ** 2)))
    ratio = err / rms if rms > 0 else float("inf")
    return Grade(n, excluded, mism, err, rms, ratio, tol, int(keep.sum()),
                 int(tokens[keep][worst]))


def _rows(out_bits, tokens):
    bits = np.asarray(out_bits)
    out = bf16_to_f64(bits).reshape(bits.shape)
    return out[np.asarray(tokens, dtype=np.int64)]


def grade_arrays(out_bits: np.ndarray, ids: np.ndarray, ref_out: np.ndarray,
                 ref_ids: np.ndarray, gaps: np.ndarray, tol: float = TOL_BF16,
                 gap_min: float = GAP_MIN) -> Grade:
    """out_bits: bf16 bits [T, H] from the device; ids [T, k] from the device;
    ref_out fp64 [T, H], ref_ids [T, k], gaps [T] from the oracle (every token)."""
    T = np.asarray(out_bits).shape[0]
    tokens = np.arange(T)
    return _core(_rows(out_bits, tokens), np.asarray(ref_out, dtype=np.float64),
                 np.asarray(ref_out, dtype=np.float64), np.asarray(ids), ref_ids, gaps, tokens,
                 tol, gap_min, False)


def grade_block_arrays(out_bits: np.ndarray, ids: np.ndarray, ref_out: np.ndarray,
                       ref_layer_out: np.ndarray, ref_ids: np.ndarray, gaps: np.ndarray,
                       tol: float = TOL_BF16, gap_min: float = GAP_MIN) -> Grade:
    """Like ``grade_arrays`` for the pre-norm block: ``max_err`` is the largest
    excess of |out - oracle| over 2^-8 |oracle|, ``rms`` the RMS of the
    oracle's layer part."""
    T = np.asarray(out_bits).shape[0]
    tokens = np.arange(T)
    return _core(_rows(out_bits, tokens), np.asarray(ref_out, dtype=np.float64),
                 np.asarray(ref_layer_out, dtype=np.float64), np.asarray(ids), ref_ids, gaps,
                 tokens, tol, gap_min, True)


def grade(out_bits: np.ndarray, ids: np.ndarray, results, tokens=None, tol: float = TOL_BF16,
          gap_min: float = GAP_MIN) -> Grade:
    """out_bits: bf16 bits [T, H] from the device; ids: int [T, k]; results:
    oracle TokenResults for ``tokens`` (default: every row, in order)."""
    results = list(results)
    tokens = np.arange(len(results)) if tokens is None else np.asarray(list(tokens), dtype=np.int64)
    if len(results) == 0:
        return Grade(0, [], [], 0.0, 0.0, float("inf"), tol, 0, -1)
    ref = np.stack([r.out for r in results])
    return _core(_rows(out_bits, tokens), ref, ref, np.asarray(ids)[tokens],
                 np.stack([r.ids for r in results]), np.array([r.gap for r in results]), tokens,
                 tol, gap_min, False)


def grade_block(out_bits: np.ndarray, ids: np.ndarray, results, tokens=None, tol: float = TOL_BF16,
                gap_min: float = GAP_MIN) -> Grade:
    """Like ``grade`` for BlockResults: ``max_err`` is the largest excess of
    |out - oracle| over the rounding allowance 2^-8 |oracle|, ``rms`` the RMS
    of the oracle's layer part (out - r)."""
    results = list(results)
    tokens = np.arange(len(results)) if tokens is None else np.asarray(list(tokens), dtype=np.int64)
    if len(results) == 0:
        return Grade(0, [], [], 0.0, 0.0, float("inf"), tol, 0, -1)
    ref = np.stack([r.out for r in results])
    moe = np.stack([r.moe.out for r in results])
    return _core(_rows(out_bits, tokens), ref, moe, np.asarray(ids)[tokens],
                 np.stack([r.ids for r in results]), np.array([r.gap for r in results]), tokens,
                 tol, gap_min, True)

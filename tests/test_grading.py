"""Pins of the parity checker (``oracle.grading``) on planted errors of known size.

Every value below is exactly representable in bf16, so the device output
passed to the checker carries exactly the planted error, and the expected
max error, RMS and ratio are closed forms.
"""

from types import SimpleNamespace

import numpy as np
import pytest

from oracle.grading import (GAP_MIN, TOL_BF16, grade, grade_arrays, grade_block,
                            grade_block_arrays)
from synth import f32_to_bf16_bits

H, K = 16, 3


def bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def reference(T=4):
    """Oracle rows of +-0.5 (RMS exactly 0.5), ids {0,1,2} per token, wide gaps."""
    ref = np.where((np.arange(T * H).reshape(T, H) % 3) == 0, -0.5, 0.5).astype(np.float64)
    ids = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    gaps = np.full(T, 1.0)
    return ref, ids, gaps


def token_results(ref, ids, gaps):
    return [SimpleNamespace(out=ref[t], ids=ids[t], gap=float(gaps[t])) for t in range(len(ref))]


def test_planted_error_gives_the_exact_ratio():
    ref, ids, gaps = reference()
    got = ref.copy()
    got[2, 5] += 2.0 ** -7          # 0.5 + 2^-7 is a bf16 value
    g = grade_arrays(bits(got), ids, ref, ids, gaps)
    assert g.n_graded == 4 and g.excluded == [] and g.id_mismatch == []
    assert g.max_err == 2.0 ** -7
    assert g.rms == 0.5
    assert g.ratio == 2.0 ** -6
    assert g.worst_token == 2
    assert g.ok                      # 0.0156 <= 0.02
    # The per-token form grades the same rows identically.
    g2 = grade(bits(got), ids, token_results(ref, ids, gaps))
    assert (g2.max_err, g2.rms, g2.ratio, g2.worst_token) == (g.max_err, g.rms, g.ratio, 2)


def test_error_above_the_tolerance_fails():
    ref, ids, gaps = reference()
    got = ref.copy()
    got[0, 1] += 2.0 ** -6           # ratio 2^-5 = 0.03125 > 0.02
    g = grade_arrays(bits(got), ids, ref, ids, gaps)
    assert g.ratio == 2.0 ** -5 and not g.ok
    assert grade_arrays(bits(got), ids, ref, ids, gaps, tol=0.04).ok


def test_id_set_mismatch_is_reported_and_fails():
    ref, ids, gaps = reference()
    dev_ids = ids.copy()
    dev_ids[1] = [0, 1, 7]           # one expert differs
    dev_ids[3] = [2, 0, 1]           # same set, other order: not a mismatch
    g = grade_arrays(bits(ref), dev_ids, ref, ids, gaps)
    assert g.id_mismatch == [1]
    assert g.max_err == 0.0 and not g.ok


def test_excluded_tokens_drop_out_of_both_checks():
    ref, ids, gaps = reference()
    got = ref.copy()
    got[3] += 1.0                    # a huge error ...
    dev_ids = ids.copy()
    dev_ids[3] = [5, 6, 7]           # ... and a wrong set, on a near-tie token
    gaps[3] = 0.5 * GAP_MIN
    g = grade_arrays(bits(got), dev_ids, ref, ids, gaps)
    assert g.excluded == [3] and g.id_mismatch == [] and g.n_graded == 3
    assert g.max_err == 0.0 and g.ok
    # Exactly at the threshold the token is graded.
    gaps[3] = GAP_MIN
    assert not grade_arrays(bits(got), dev_ids, ref, ids, gaps).ok


def test_all_excluded_or_empty_fails():
    ref, ids, gaps = reference()
    g = grade_arrays(bits(ref), ids, ref, ids, np.zeros(len(ref)))
    assert g.n_graded == 0 and len(g.excluded) == len(ref) and not g.ok
    assert not grade(bits(ref), ids, []).ok
    assert not grade_block(bits(ref), ids, []).ok


def test_sampled_tokens_map_to_their_rows():
    ref, ids, gaps = reference(T=6)
    got = ref.copy()
    got[4, 0] += 2.0 ** -7
    sample = [1, 4]
    res = token_results(ref, ids, gaps)
    g = grade(bits(got), ids, [res[t] for t in sample], tokens=sample)
    assert g.worst_token == 4 and g.max_err == 2.0 ** -7 and g.n_graded == 2
    g = grade(bits(got), ids, [res[t] for t in [0, 5]], tokens=[0, 5])
    assert g.max_err == 0.0


def test_block_grading_allows_the_rounding_of_the_sum():
    """out = r + layer: |err| up to 2^-8 |oracle out| is the bf16 rounding of
    the sum and is not counted; the RMS is that of the layer part."""
    T = 2
    r = np.full((T, H), 16.0)
    layer = np.where(np.arange(T * H).reshape(T, H) % 2 == 0, 0.25, -0.25)
    ref = r + layer                   # 16.25 / 15.75 (bf16 spacing 2^-3 there)
    ids = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    gaps = np.ones(T)
    got = ref.copy()
    got[0, 0] += 2.0 ** -3            # one spacing: 0.125 - 16.25 / 256 beyond the allowance
    g = grade_block_arrays(bits(got), ids, ref, layer, ids, gaps)
    assert g.rms == 0.25
    assert g.max_err == pytest.approx(0.125 - 16.25 / 256, abs=0)
    assert g.ratio == pytest.approx((0.125 - 16.25 / 256) / 0.25, rel=1e-15)
    assert not g.ok
    # Only the part of an error beyond the allowance counts: 2^-4 above
    # 15.75 exceeds 15.75 / 256 by 0.00098.
    got = ref.copy()
    got[1, 3] = 15.75 + 2.0 ** -4
    g = grade_block_arrays(bits(got), ids, ref, layer, ids, gaps)
    assert g.max_err == pytest.approx(2.0 ** -4 - 15.75 / 256, abs=0)
    assert g.ok
    res = [SimpleNamespace(out=ref[t], ids=ids[t], gap=1.0, moe=SimpleNamespace(out=layer[t]))
           for t in range(T)]
    g2 = grade_block(bits(got), ids, res)
    assert (g2.max_err, g2.rms) == (g.max_err, g.rms)


def test_default_tolerance_is_the_north_star_bf16_bound():
    assert TOL_BF16 == 2e-2 and GAP_MIN == 1e-5

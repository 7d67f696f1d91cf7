"""Pins of the pre-norm block oracle (RMSNorm, bf16 rounding, residual add).

Each test checks a consequence that a plausible mistake would break: a sum of
squares instead of a mean, eps outside the square root, gamma dropped or
applied to the wrong element, the residual dropped or subtracted, the norm's
bf16 rounding done with truncation or ties away from zero, or the MoE fed the
un-normalised input.
"""

import math

import numpy as np
import pytest

from oracle import OracleLayer, bf16_to_f64, moe_token
from oracle.block import block_forward, block_token, f64_to_bf16_bits, rmsnorm
from synth import SyntheticLayer, LayerShape, f32_to_bf16_bits, make_x


def bits(a):
    a = np.asarray(a, dtype=np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_to_f64(b), a.astype(np.float64)), "value not bf16-exact"
    return b


def small_layer(H=4, E=4, k=2, I=2, seed=3, zero_w2=False):
    rng = np.random.default_rng(seed)
    q = lambda *s: np.round(rng.standard_normal(s) * 8) / 16   # bf16-exact
    ex = {}
    for e in range(-1, E):
        w13, w2 = q(2 * I, H), q(H, I)
        if zero_w2:
            w2 = np.zeros_like(w2)
        ex[e] = (bits(w13), bits(w2))
    return OracleLayer(hidden=H, n_experts=E, top_k=k, inter=I, router_w_bits=bits(q(E, H)),
                       router_b=None, expert_raw=lambda e: ex[e])


# ---------------------------------------------------------------- bf16 rounding

@pytest.mark.parametrize("v,expect", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                    # halfway, ties to the even neighbour (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),                # halfway, ties to the even neighbour (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),       # just past halfway rounds up
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),       # just short of halfway rounds down
    (-2.5, 0xC020),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0 ** -133, 0x0001),                        # smallest subnormal
    (2.0 ** -134, 0x0000),                        # half of it: tie to even (zero)
    (3 * 2.0 ** -134, 0x0002),                    # 1.5 spacings: tie to even (2)
    (2.0 ** -126, 0x0080),                        # smallest normal
    (3.3895313892515355e38, 0x7F7F),              # largest finite bf16
    (3.4e38, 0x7F80),                             # past the last midpoint: infinity
    (1.2, 0x3F9A),                                # 1.2 * 128 = 153.6 -> 154
    (1.6, 0x3FCD),                                # 1.6 * 128 = 204.8 -> 205
])
def test_bf16_rounding_hand_values(v, expect):
    assert int(f64_to_bf16_bits(np.array([v]))[0]) == expect


def test_bf16_rounding_every_midpoint():
    """For every pair of adjacent finite non-negative bf16 values: their exact
    midpoint goes to the one with an even pattern, and points just either
    side of it go to the nearer value."""
    lo = np.arange(0x0000, 0x7F7F, dtype=np.uint16)
    hi = lo + np.uint16(1)
    a, b = bf16_to_f64(lo), bf16_to_f64(hi)
    mid = (a + b) / 2                      # exact in fp64
    eps = (b - a) * 2.0 ** -20
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(f64_to_bf16_bits(mid), even)
    assert np.array_equal(f64_to_bf16_bits(mid + eps), hi)
    assert np.array_equal(f64_to_bf16_bits(mid - eps), lo)
    # and the negatives mirror them with the sign bit set
    assert np.array_equal(f64_to_bf16_bits(-mid), even | np.uint16(0x8000))


def test_bf16_rounding_agrees_with_fp32_bit_trick():
    """On fp32-exact inputs, one-step rounding equals the fp32 bit-pattern
    rounding of the input generators (an independent implementation)."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(np.float32)
    assert np.array_equal(f64_to_bf16_bits(v.astype(np.float64)), f32_to_bf16_bits(v))


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_worked_example():
    # mean of squares of (3, 4) = 12.5; 3 / sqrt(12.5) = 0.84852813742385702, 4 / sqrt(12.5) = 1.1313708498984760
    n = rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 1.0]), eps=0.0)
    np.testing.assert_allclose(n, [0.84852813742385702, 1.1313708498984760], rtol=1e-15)
    # gamma scales element by element, in place
    n = rmsnorm(np.array([3.0, 4.0]), np.array([2.0, 0.5]), eps=0.0)
    np.testing.assert_allclose(n, [1.6970562748477140, 0.56568542494923802], rtol=1e-15)


def test_rmsnorm_eps_inside_the_root():
    # constant 1e-3 over 2048 elements: mean square 1e-6; with eps 1e-6 the divisor is sqrt(2e-6)
    n = rmsnorm(np.full(2048, 1e-3), np.ones(2048), eps=1e-6)
    np.testing.assert_allclose(n, np.full(2048, 1 / math.sqrt(2)), rtol=1e-14)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(5)
    r = rng.standard_normal((7, 2048)) * 13.0
    n = rmsnorm(r, np.ones(2048), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(rmsnorm(r * 1e3, np.ones(2048), eps=0.0), n, rtol=1e-12)
    # rows are normalised independently
    np.testing.assert_allclose(rmsnorm(r[3], np.ones(2048), eps=0.0), n[3], rtol=0)


# ---------------------------------------------------------------- the block

def test_block_worked_example():
    """H = 4: r = (3, 4, 0, 0) has RMS 2.5, so with gamma = 1 and eps = 0 the
    normalised input is (1.2, 1.6, 0, 0), rounded to bf16 (1.203125, 1.6015625).
    Shared expert only (routed_scale 0): gate row picks n[0], up row picks
    n[1], and w2 maps the single h to output 0 with weight 2, so
    out = r + (2 * silu(1.203125) * 1.6015625, 0, 0, 0)."""
    H, I, E = 4, 1, 2
    w13 = np.zeros((2, H)); w13[0, 0] = 1.0; w13[1, 1] = 1.0
    w2 = np.zeros((H, I)); w2[0, 0] = 2.0
    ex = {e: (bits(w13), bits(w2)) for e in (-1, 0, 1)}
    L = OracleLayer(hidden=H, n_experts=E, top_k=1, inter=I, router_w_bits=bits(np.zeros((E, H))),
                    router_b=None, expert_raw=lambda e: ex[e])
    r = bits([3.0, 4.0, 0.0, 0.0])
    res = block_token(L, r, bits(np.ones(H)), eps=0.0, routed_scale=0.0)
    assert res.normed_bits.tolist() == [0x3F9A, 0x3FCD, 0, 0]
    g = 1.203125
    y0 = 2 * g / (1 + math.exp(-g)) * 1.6015625
    np.testing.assert_allclose(res.out, [3.0 + y0, 4.0, 0.0, 0.0], rtol=1e-15, atol=0)


def test_block_zero_gamma_returns_the_residual():
    L = small_layer()
    r = bits(np.array([[1.5, -2.0, 0.25, 8.0], [0.0, 0.0, 0.0, 0.0]]))
    for t, res in enumerate(block_forward(L, r, bits(np.zeros(4)))):
        assert not np.any(res.normed_bits & np.uint16(0x7FFF))
        np.testing.assert_array_equal(res.out, bf16_to_f64(r[t]))


def test_block_zero_down_projections_return_the_residual():
    L = small_layer(zero_w2=True)
    r = bits(np.array([[1.5, -2.0, 0.25, 8.0]]))
    res = block_forward(L, r, bits([1.0, 0.5, 2.0, -1.0]))[0]
    np.testing.assert_array_equal(res.out, bf16_to_f64(r[0]))


def test_block_reduces_to_the_layer_on_unit_rms_input():
    """Entries of magnitude 1 have RMS exactly 1: with gamma = 1 and eps = 0 the
    norm is the identity, so out - r is the layer's output on r itself."""
    S = SyntheticLayer(seed=2, shape=LayerShape(hidden=256, n_experts=16, top_k=4, inter=64))
    w13, w2 = S.routed_banks(threads=2)
    sh = S.shared()
    L = OracleLayer(hidden=256, n_experts=16, top_k=4, inter=64, router_w_bits=S.router_w(),
                    router_b=None, expert_raw=lambda e: sh if e < 0 else (w13[e], w2[e]))
    rng = np.random.default_rng(9)
    r = bits(np.where(rng.random(256) < 0.5, -1.0, 1.0))
    res = block_token(L, r, bits(np.ones(256)), eps=0.0)
    assert np.array_equal(res.normed_bits, r)
    ref = moe_token(L, r)
    np.testing.assert_array_equal(res.out, bf16_to_f64(r) + ref.out)
    assert res.ids.tolist() == ref.ids.tolist()


def test_block_routes_on_the_normalised_input():
    """Scaling r scales the residual but leaves the MoE part alone (the norm
    removes the scale before the router sees it) as long as eps is 0."""
    L = small_layer(seed=8)
    r = bits([1.0, -3.0, 0.5, 2.0])
    r4 = bits([4.0, -12.0, 2.0, 8.0])
    g = bits([1.0, 2.0, 0.5, 1.0])
    a = block_token(L, r, g, eps=0.0)
    b = block_token(L, r4, g, eps=0.0)
    assert np.array_equal(a.normed_bits, b.normed_bits)
    np.testing.assert_allclose(b.out - bf16_to_f64(r4), a.out - bf16_to_f64(r), rtol=0, atol=1e-13)


def test_block_forward_is_per_token():
    S = SyntheticLayer(seed=4, shape=LayerShape(hidden=128, n_experts=8, top_k=2, inter=32))
    w13, w2 = S.routed_banks(threads=2)
    sh = S.shared()
    L = OracleLayer(hidden=128, n_experts=8, top_k=2, inter=32, router_w_bits=S.router_w(),
                    router_b=None, expert_raw=lambda e: sh if e < 0 else (w13[e], w2[e]))
    R = make_x(5, hidden=128, seed=4, x_seed=1)
    g = f32_to_bf16_bits(np.linspace(0.5, 1.5, 128).astype(np.float32))
    allr = block_forward(L, R, g)
    for t in (0, 3, 4):
        one = block_token(L, R[t], g)
        np.testing.assert_array_equal(allr[t].out, one.out)


def test_grade_block_rounding_allowance():
    """The block grade accepts the stored sum's own bf16 rounding and rejects
    an error in the layer part above the tolerance, however large r is."""
    from oracle.grading import grade_block
    L = small_layer(seed=12)
    r = bits(np.array([[300.0, -2.0, 0.25, 8.0], [1.0, 2.0, 3.0, 4.0]]))
    res = block_forward(L, r, bits([1.0, 0.5, 2.0, -1.0]))
    ids = np.stack([x.ids for x in res])
    good = f64_to_bf16_bits(np.stack([x.out for x in res]))
    assert grade_block(good, ids, res).ok
    bad = np.stack([x.out for x in res])
    bad[0, 1] += 0.05 * np.sqrt(np.mean(np.stack([x.moe.out for x in res]) ** 2))
    assert not grade_block(f64_to_bf16_bits(bad), ids, res).ok

"""Pins of the low-latency decode path's oracle (``oracle.decoder``): the
attention output projection, the rounded residual adds, and the next
layer's norm around the pre-norm MoE block, against closed forms, hand-worked
values, brute force and reductions to the already pinned block oracle."""

import numpy as np
import pytest

from oracle import OracleLayer, bf16_to_f64
from oracle.block import block_forward, f64_to_bf16_bits
from oracle.decoder import decoder_forward, decoder_token, o_proj
from synth import LayerShape, SyntheticLayer, f32_to_bf16_bits, make_residual

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

H, E, K, I, W = 32, 8, 3, 16, 64


def tiny(seed=5):
    syn = SyntheticLayer(seed, LayerShape(hidden=H, n_experts=E, top_k=K, inter=I))
    L = OracleLayer(H, E, K, I, syn.router_w(), None, syn.expert)
    return syn, L


def bits(a):
    a = np.asarray(a, dtype=np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_to_f64(b).reshape(a.shape), a.astype(np.float64))
    return b


def rand_bits(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits((rng.standard_normal(int(np.prod(shape))) * std).astype(np.float32)).reshape(shape)


def test_o_proj_matches_brute_force_double_loop():
    wo = rand_bits((H, W), 1, 0.05)
    a = rand_bits((W,), 2)
    wf, af = bf16_to_f64(wo).reshape(H, W), bf16_to_f64(a)
    brute = np.array([sum(wf[i, j] * af[j] for j in range(W)) for i in range(H)])
    np.testing.assert_allclose(o_proj(wf, a), brute, rtol=1e-13, atol=1e-15)
    # Linear in a: o(a + b) = o(a) + o(b) for bf16-exact a, b, a + b.
    b = bits(np.ones(W, np.float32) * 0.5)
    a2 = bits(np.full(W, 0.25, np.float32))
    np.testing.assert_allclose(o_proj(wf, bits(np.full(W, 0.75, np.float32))),
                               o_proj(wf, b) + o_proj(wf, a2), rtol=1e-14)


def test_worked_example_of_the_residual_add_and_its_rounding():
    """Wo = [I | 0]: r1 = bf16(r + a[:H]).  In [1, 2) the bf16 spacing is
    2^-7: 1 + 2^-8 is a midpoint and ties to the even 1.0, 1 + 2^-7 + 2^-8
    ties up to the even 1 + 2^-6; in [2, 4) the spacing is 2^-6, so
    3 + 2^-6 is exact; -2 + 0.5 = -1.5 is exact."""
    syn, L = tiny()
    wo = np.zeros((H, W), np.float32)
    wo[np.arange(H), np.arange(H)] = 1.0
    r = np.zeros(H, np.float32)
    a = np.zeros(W, np.float32)
    r[0], a[0] = 1.0, 2.0 ** -8
    r[1], a[1] = 1.0 + 2.0 ** -7, 2.0 ** -8
    r[2], a[2] = 3.0, 2.0 ** -6
    r[3], a[3] = -2.0, 0.5
    res = decoder_token(L, bf16_to_f64(bits(wo)).reshape(H, W), bits(a), bits(r),
                        syn.norm_weight())
    got = bf16_to_f64(res.r1_bits)
    assert got[0] == 1.0
    assert got[1] == 1.0 + 2.0 ** -6
    assert got[2] == 3.0 + 2.0 ** -6       # spacing at 2..4 is 2^-6: exact
    assert got[3] == -1.5
    assert res.r1_f64[0] == 1.0 + 2.0 ** -8   # the unrounded sum is kept


def test_zero_projection_reduces_to_the_block_on_r():
    syn, L = tiny()
    T = 5
    rb = make_residual(T, hidden=H, seed=5, x_seed=1)
    gamma = syn.norm_weight()
    for wo, attn in ((np.zeros((H, W), np.uint16), rand_bits((T, W), 3)),
                     (rand_bits((H, W), 4, 0.05), np.zeros((T, W), np.uint16))):
        res = decoder_forward(L, wo, attn, rb, gamma)
        ref = block_forward(L, rb, gamma)
        for t in range(T):
            assert np.array_equal(res[t].r1_bits, rb[t])
            assert res[t].ids.tolist() == ref[t].ids.tolist()
            np.testing.assert_array_equal(res[t].out, ref[t].out)
            np.testing.assert_array_equal(res[t].r2_bits, f64_to_bf16_bits(ref[t].out))


def test_r1_is_the_rounded_sum_and_feeds_the_block():
    syn, L = tiny()
    T = 4
    wo = rand_bits((H, W), 6, 0.05)
    attn = rand_bits((T, W), 7)
    rb = make_residual(T, hidden=H, seed=5, x_seed=2)
    gamma = syn.norm_weight()
    res = decoder_forward(L, wo, attn, rb, gamma)
    wf = bf16_to_f64(wo).reshape(H, W)
    r1 = np.stack([f64_to_bf16_bits(bf16_to_f64(rb[t]) + wf @ bf16_to_f64(attn[t])) for t in range(T)])
    ref = block_forward(L, r1, gamma)
    for t in range(T):
        np.testing.assert_array_equal(res[t].r1_bits, r1[t])
        np.testing.assert_array_equal(res[t].out, ref[t].out)
        assert res[t].gap == ref[t].gap


def test_next_norm_closed_forms():
    """MoE output zero (routed_scale 0, shared w2 zero): r2 = r1.  With r1
    entries +-c, eps = 0 and gamma_next = 1, n2 = +-1 exactly; gamma_next = 0
    gives n2 = 0."""
    syn, _ = tiny()
    ex = {e: syn.expert(e) for e in range(E)}
    ex[-1] = (syn.expert(-1)[0], np.zeros((H, I), np.uint16))
    L = OracleLayer(H, E, K, I, syn.router_w(), None, lambda e: ex[e])
    wo = np.zeros((H, W), np.uint16)
    sign = np.where(np.arange(H) % 3 == 0, -1.0, 1.0).astype(np.float32)
    r = bits(sign * 0.375)
    attn = np.zeros(W, np.uint16)
    one = bits(np.ones(H, np.float32))
    res = decoder_token(L, bf16_to_f64(wo).reshape(H, W), attn, r, syn.norm_weight(),
                        gamma_next_bits=one, eps=0.0, routed_scale=0.0)
    np.testing.assert_array_equal(res.r2_bits, r)
    np.testing.assert_array_equal(bf16_to_f64(res.n2_bits), sign.astype(np.float64))
    res0 = decoder_token(L, bf16_to_f64(wo).reshape(H, W), attn, r, syn.norm_weight(),
                         gamma_next_bits=np.zeros(H, np.uint16), routed_scale=0.0)
    assert not np.any(res0.n2_bits & np.uint16(0x7FFF))


def test_next_norm_is_the_rmsnorm_of_the_rounded_r2():
    """(3, 4, 0, ..., 0) scaled: the RMSNorm closed form 3/sqrt(25/H), 4/sqrt(25/H)."""
    syn, _ = tiny()
    ex = {e: syn.expert(e) for e in range(E)}
    ex[-1] = (syn.expert(-1)[0], np.zeros((H, I), np.uint16))
    L = OracleLayer(H, E, K, I, syn.router_w(), None, lambda e: ex[e])
    r = np.zeros(H, np.float32)
    r[0], r[1] = 3.0, 4.0
    res = decoder_token(L, np.zeros((H, W)), np.zeros(W, np.uint16), bits(r), syn.norm_weight(),
                        gamma_next_bits=bits(np.ones(H, np.float32)), eps=0.0, routed_scale=0.0)
    s = np.sqrt(25.0 / H)
    np.testing.assert_allclose(res.n2_f64[:2], [3.0 / s, 4.0 / s], rtol=1e-15)
    assert not np.any(res.n2_f64[2:])

"""Pins of the expert-grouped oracle (``oracle.grouped``) against the per-token
oracle, which is itself pinned by closed forms, brute force and invariants
(``test_oracle_pins.py``, ``test_oracle_block.py``, ``test_oracle_dense.py``).

The grouped form is the same arithmetic regrouped per expert, so each token's
output must agree with the per-token oracle to fp64 rounding (a few units in
the last place), its ids exactly, and its weights and gap to ~1e-15.
"""

import numpy as np
import pytest

from oracle import OracleLayer, moe_forward, route_all
from oracle.block import block_forward
from oracle.dense import DenseMLP, mlp_block_forward, mlp_forward
from oracle.grouped import (block_forward_grouped, mlp_forward_batched, moe_forward_grouped,
                            route_rows)
from oracle.moe import bf16_to_f64
from synth import LayerShape, SyntheticDenseMLP, SyntheticLayer, make_residual, make_x

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.fixture(scope="module")
def flint_layer():
    syn = SyntheticLayer(0)
    syn.routed_banks()
    return syn


def close(a, b, rel=1e-12):
    scale = float(np.sqrt(np.mean(np.asarray(b) ** 2)))
    assert np.max(np.abs(np.asarray(a) - np.asarray(b))) <= rel * scale


@pytest.mark.parametrize("bias,T,x_seed", [(False, 48, 5), (True, 64, 6)])
def test_grouped_layer_matches_per_token_oracle(flint_layer, bias, T, x_seed):
    """Full Flint-shape layer (256 experts, H 2048, I 512), every token; with
    the router bias, experts hit by many tokens are grouped."""
    syn = flint_layer
    L = OracleLayer(2048, 256, 6, 512, syn.router_w(), syn.router_bias() if bias else None,
                    syn.expert)
    xb = make_x(T, seed=0, x_seed=x_seed)
    G = moe_forward_grouped(L, xb)
    if bias:
        assert np.bincount(G.ids.ravel(), minlength=256).max() >= 8   # real groups
    for t, r in enumerate(moe_forward(L, xb)):
        assert G.ids[t].tolist() == r.ids.tolist()
        assert abs(G.gaps[t] - r.gap) <= 1e-15
        np.testing.assert_allclose(G.weights[t], r.weights, rtol=1e-14, atol=0)
        np.testing.assert_allclose(G.logits[t], r.logits, rtol=0, atol=1e-13)
        close(G.out[t], r.out)


def test_grouped_layer_options_match(flint_layer):
    """renormalize off and a routed scale, on a smaller expert count."""
    syn = SyntheticLayer(4, LayerShape(n_experts=16))
    L = OracleLayer(2048, 16, 6, 512, syn.router_w(), None, syn.expert)
    xb = make_x(12, seed=4, x_seed=1)
    for renorm, scale in ((False, 1.0), (True, 2.5), (True, 0.0)):
        G = moe_forward_grouped(L, xb, renormalize=renorm, routed_scale=scale)
        for t, r in enumerate(moe_forward(L, xb, renormalize=renorm, routed_scale=scale)):
            np.testing.assert_allclose(G.weights[t], r.weights, rtol=1e-14, atol=0)
            close(G.out[t], r.out)


def test_route_rows_matches_route_all_and_breaks_ties_low(flint_layer):
    syn = flint_layer
    L = OracleLayer(2048, 256, 6, 512, syn.router_w(), syn.router_bias(), syn.expert)
    xb = make_x(32, seed=0, x_seed=9)
    ids, w, gaps, Z = route_rows(L, bf16_to_f64(xb).reshape(32, 2048))
    ids2, w2, gaps2, Z2 = route_all(L, xb)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-14, atol=0)
    np.testing.assert_allclose(gaps, gaps2, rtol=0, atol=1e-15)
    # All-zero router: every score is 1/2, the picks are experts 0..5 in order.
    Z0 = OracleLayer(2048, 256, 6, 512, np.zeros((256, 2048), np.uint16), None, syn.expert)
    ids0, w0, g0, _ = route_rows(Z0, np.ones((3, 2048)))
    assert ids0.tolist() == [list(range(6))] * 3
    np.testing.assert_array_equal(w0, np.full((3, 6), 1.0 / 6))
    np.testing.assert_array_equal(g0, np.zeros(3))


def test_grouped_block_matches_per_token_oracle(flint_layer):
    syn = flint_layer
    L = OracleLayer(2048, 256, 6, 512, syn.router_w(), None, syn.expert)
    rb = make_residual(24, seed=0, x_seed=2)
    gamma = syn.norm_weight()
    G = block_forward_grouped(L, rb, gamma)
    for t, r in enumerate(block_forward(L, rb, gamma)):
        np.testing.assert_array_equal(G.normed_bits[t], r.normed_bits)
        assert G.ids[t].tolist() == r.ids.tolist()
        close(G.layer_out[t], r.moe.out)
        close(G.out[t] - bf16_to_f64(rb[t]), r.out - bf16_to_f64(rb[t]))


@pytest.mark.parametrize("inter", [512, 1536])
def test_batched_dense_mlp_matches_per_token_oracle(inter):
    S = SyntheticDenseMLP(1, inter)
    xb = make_x(40, seed=1, x_seed=3)
    y = mlp_forward_batched(S.w13(), S.w2(), xb, 2048, inter, chunk=16)
    M = DenseMLP(2048, inter, S.w13(), S.w2())
    for t, (o, _) in enumerate(mlp_forward(M, xb)):
        close(y[t], o)
    rb = make_residual(10, seed=1, x_seed=4)
    out, part = mlp_forward_batched(S.w13(), S.w2(), rb, 2048, inter, gamma_bits=S.norm_weight())
    for t, r in enumerate(mlp_block_forward(M, rb, S.norm_weight())):
        close(part[t], r.mlp_out)
        close(out[t] - bf16_to_f64(rb[t]), r.out - bf16_to_f64(rb[t]))

"""Pins of the CPU oracle against closed forms, brute force and invariants.

None of these re-types the oracle's formula: each checks a consequence that a
plausible mistake (a dropped term, a wrong sign or index, a transposed
operand, swapped gate/up halves, a wrong tie-break) would break.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import (OracleLayer, bf16_to_f64, bucket, expert_forward, moe_forward,
                    moe_token, route_all, router_logits, routing_weights,
                    select_topk, sigmoid, silu)
from synth import LayerShape, SyntheticLayer, f32_to_bf16_bits, make_x

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bits(a):
    """bf16 bits of values that are exactly representable in bf16."""
    a = np.asarray(a, dtype=np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_to_f64(b), a.astype(np.float64)), "value not bf16-exact"
    return b


def layer_from_arrays(router, experts, shared, top_k, bias=None):
    """OracleLayer over explicit float arrays (bf16-exact values)."""
    E, H = np.asarray(router).shape
    I = np.asarray(shared[1]).shape[1]
    ex = {e: (bits(w13), bits(w2)) for e, (w13, w2) in enumerate(experts)}
    ex[-1] = (bits(shared[0]), bits(shared[1]))
    return OracleLayer(hidden=H, n_experts=E, top_k=top_k, inter=I,
                       router_w_bits=bits(router),
                       router_b=None if bias is None else np.asarray(bias, np.float32),
                       expert_raw=lambda e: ex[e])


def tiny_seeded(seed=3, H=32, E=8, k=3, I=16, with_bias=False):
    syn = SyntheticLayer(seed, LayerShape(hidden=H, n_experts=E, top_k=k, inter=I))
    return syn, OracleLayer(hidden=H, n_experts=E, top_k=k, inter=I,
                            router_w_bits=syn.router_w(),
                            router_b=syn.router_bias() if with_bias else None,
                            expert_raw=syn.expert)


# ---------------------------------------------------------------- elementwise

def test_bf16_decode_closed_forms():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x3E80: 0.25,
             0x4049: 3.140625, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x8080: -(2.0 ** -126)}
    for b, v in cases.items():
        assert bf16_to_f64(np.array([b], np.uint16))[0] == v


def test_sigmoid_closed_forms():
    assert sigmoid(0.0) == 0.5
    assert sigmoid(math.log(3.0)) == pytest.approx(0.75, abs=1e-15)
    assert sigmoid(-math.log(3.0)) == pytest.approx(0.25, abs=1e-15)
    z = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(sigmoid(z) + sigmoid(-z), 1.0, atol=1e-15)
    assert np.all(np.diff(sigmoid(z)) > 0)


def test_silu_closed_forms():
    assert silu(0.0) == 0.0
    assert silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), abs=1e-15)
    g = np.linspace(-12, 12, 97)
    # silu(-g) = -g * sigma(-g) = -g * (1 - sigma(g)) = silu(g) - g
    np.testing.assert_allclose(silu(-g), silu(g) - g, atol=1e-13)
    assert silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(silu(-40.0)) < 1e-15


# ---------------------------------------------------------------- selection

def _brute_topk(s, k):
    """Exhaustive search: maximise the sum, ties to the lexicographically
    smallest index set; then rank by score, ties to lower index."""
    best = None
    for sub in itertools.combinations(range(len(s)), k):
        key = (sum(s[i] for i in sub), tuple(-i for i in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    sub = best[1]
    return sorted(sub, key=lambda i: (-s[i], i))


@pytest.mark.parametrize("trial", range(12))
def test_topk_brute_force_all_k(trial):
    rng = np.random.default_rng(100 + trial)
    E = 8
    if trial % 3 == 0:
        s = rng.choice([0.1, 0.5, 0.9], size=E).astype(np.float64)  # many ties
    else:
        s = sigmoid(rng.standard_normal(E))
    for k in range(1, E + 1):
        ids, gap = select_topk(s, k)
        assert list(ids) == _brute_topk(list(s), k)
        sel = set(ids.tolist())
        uns = [e for e in range(E) if e not in sel]
        assert all(s[a] >= s[b] for a in sel for b in uns)
        if uns:
            assert gap == pytest.approx(min(s[a] for a in sel) - max(s[b] for b in uns), abs=0)
        else:
            assert gap == math.inf


def test_topk_all_equal_scores_pick_lowest_indices():
    ids, gap = select_topk(np.full(256, 0.5), 6)
    assert ids.tolist() == [0, 1, 2, 3, 4, 5]
    assert gap == 0.0


def test_routing_weights_renorm_and_scale():
    s = sigmoid(np.array([0.3, -1.2, 2.0, 0.0, 5.0]))
    ids = np.array([4, 2, 0])
    w = routing_weights(s, ids, True, 1.0)
    assert w.sum() == pytest.approx(1.0, abs=1e-15)
    assert w[0] / w[1] == pytest.approx(s[4] / s[2], rel=1e-15)
    w_off = routing_weights(s, ids, False, 1.0)
    np.testing.assert_array_equal(w_off, s[ids])
    w_sc = routing_weights(s, ids, True, 2.5)
    np.testing.assert_allclose(w_sc, 2.5 * w, rtol=1e-15)


# ---------------------------------------------------------------- GEMV steps

def test_router_gemv_one_hot_rows():
    """Router row e = one-hot at column p(e) => z_e = x[p(e)] (+ b_e).  E != H
    and an irregular p catch a transposed weight or a wrong axis."""
    H, E = 12, 5
    p = [7, 0, 11, 3, 3]
    W = np.zeros((E, H))
    for e, c in enumerate(p):
        W[e, c] = 2.0 ** -e
    x = np.arange(1, H + 1, dtype=np.float64) * 0.25
    b = np.array([0.5, -1.0, 0.0, 2.0, -0.25])
    z = router_logits(x, W, None)
    np.testing.assert_array_equal(z, [x[c] * 2.0 ** -e for e, c in enumerate(p)])
    np.testing.assert_array_equal(router_logits(x, W, b), z + b)


def test_expert_structured_closed_form():
    """gate row i = alpha_i e_{a_i}, up row i = beta_i e_{b_i}, W2 row j = e_{c_j}:
    h_i = silu(alpha_i x[a_i]) * beta_i x[b_i] and y_j = h[c_j].  Swapping the
    gate and up halves, or transposing W2, changes the result."""
    H, I = 10, 4
    a, b_, c = [3, 0, 9, 5], [1, 1, 7, 2], [2, 0, 3, 3, 1, 0, 2, 1, 0, 3]
    alpha, beta = [1.0, -2.0, 0.5, 4.0], [0.75, 1.5, -1.0, 2.0]
    w13 = np.zeros((2 * I, H))
    for i in range(I):
        w13[i, a[i]] = alpha[i]
        w13[I + i, b_[i]] = beta[i]
    w2 = np.zeros((H, I))
    for j in range(H):
        w2[j, c[j]] = 1.0
    x = np.array([0.5, -1.25, 2.0, 1.0, -0.5, 3.0, 0.25, -2.0, 1.5, -0.75])
    y, h = expert_forward(w13, w2, x, I)
    h_exp = [alpha[i] * x[a[i]] / (1 + math.exp(-alpha[i] * x[a[i]])) * beta[i] * x[b_[i]]
             for i in range(I)]
    np.testing.assert_allclose(h, h_exp, rtol=1e-14)
    np.testing.assert_allclose(y, [h_exp[cj] for cj in c], rtol=1e-14)


# ---------------------------------------------------------------- whole layer

def test_worked_example_closed_form():
    """A 4-expert, top-2 layer worked by hand.  Logits come out 0, 1, 1, -1 so
    experts 1 and 2 tie on score and both beat expert 0; renormalised weights
    are 1/2 each.  With a = silu(1), b = silu(2), c = silu(-1) the output is
    [b/2 + a, c + a/2, a/2, b/2 - c - a/2]."""
    e = np.eye(4)
    router = np.stack([np.zeros(4), e[0], 0.5 * e[1], e[2]])
    ones = (np.ones((4, 4)), np.ones((4, 2)))
    ex1 = (np.stack([e[0], 0.5 * e[1], e[1], e[2]]),
           np.array([[1, 0], [0, 1], [1, 1], [0, 0]], dtype=float))
    ex2 = (np.stack([2.0 * e[3], np.zeros(4), e[0], e[1]]),
           np.array([[0, 0], [2, 0], [0, 0], [-1, 0]], dtype=float))
    shared = (np.stack([e[1], e[2], e[3], e[0]]),
              np.array([[1, 0], [0, 1], [0, 0], [1, -1]], dtype=float))
    layer = layer_from_arrays(router, [ones, ex1, ex2, ones], shared, top_k=2)
    x = bits([1.0, 2.0, -1.0, 0.5])
    r = moe_token(layer, x)
    a = 1 / (1 + math.exp(-1))
    b = 2 / (1 + math.exp(-2))
    c = -1 / (1 + math.exp(1))
    assert r.ids.tolist() == [1, 2]
    np.testing.assert_allclose(r.weights, [0.5, 0.5], rtol=1e-15)
    assert r.gap == pytest.approx(1 / (1 + math.exp(-1)) - 0.5, rel=1e-14)
    np.testing.assert_allclose(r.out, [b / 2 + a, c + a / 2, a / 2, b / 2 - c - a / 2],
                               rtol=1e-13, atol=1e-15)


def test_zero_routed_scale_gives_shared_expert_alone():
    syn, layer = tiny_seeded()
    X = make_x(5, 32, seed=3, x_seed=1)
    w13, w2 = (bf16_to_f64(a) for a in syn.shared())
    for t, r in enumerate(moe_forward(layer, X, routed_scale=0.0)):
        y, _ = expert_forward(w13.reshape(32, 32), w2.reshape(32, 16), bf16_to_f64(X[t]), 16)
        np.testing.assert_allclose(r.out, y, rtol=0, atol=0)


def test_zero_routed_w2_gives_shared_expert_alone():
    syn, layer = tiny_seeded()
    X = make_x(4, 32, seed=3, x_seed=2)
    z2 = np.zeros((32, 16), np.uint16)
    zero_layer = OracleLayer(32, 8, 3, 16, layer.router_w_bits, None,
                             lambda e: syn.expert(e) if e < 0 else (syn.expert(e)[0], z2))
    ref = moe_forward(layer, X, routed_scale=0.0)
    for r0, r in zip(ref, moe_forward(zero_layer, X)):
        np.testing.assert_allclose(r.out, r0.out, rtol=0, atol=1e-15)


def test_identical_experts_renormalised_double_the_expert():
    """All routed experts and the shared expert equal E_0 with renorm on:
    out = E_0(x) + (sum_j w_j) E_0(x) = 2 E_0(x), whatever the routing."""
    syn, base = tiny_seeded(seed=5)
    same = syn.expert(0)
    layer = OracleLayer(32, 8, 3, 16, base.router_w_bits, None, lambda e: same)
    X = make_x(6, 32, seed=5, x_seed=0)
    w13, w2 = bf16_to_f64(same[0]).reshape(32, 32), bf16_to_f64(same[1]).reshape(32, 16)
    for t, r in enumerate(moe_forward(layer, X)):
        y, _ = expert_forward(w13, w2, bf16_to_f64(X[t]), 16)
        np.testing.assert_allclose(r.out, 2 * y, rtol=1e-12, atol=1e-14)
        assert r.weights.sum() == pytest.approx(1.0, abs=1e-15)


def test_permuting_experts_permutes_ids_only():
    syn, layer = tiny_seeded(seed=9, with_bias=True)
    perm = np.random.default_rng(1).permutation(8)        # new index n holds old expert perm[n]
    inv = np.argsort(perm)
    Wr = syn.router_w()[perm]
    pl = OracleLayer(32, 8, 3, 16, Wr, syn.router_bias()[perm],
                     lambda e: syn.expert(e if e < 0 else int(perm[e])))
    X = make_x(7, 32, seed=9, x_seed=3)
    for r0, r1 in zip(moe_forward(layer, X), moe_forward(pl, X)):
        assert [int(perm[i]) for i in r1.ids] == r0.ids.tolist()
        assert inv[r0.ids].tolist() == r1.ids.tolist()
        np.testing.assert_allclose(r1.out, r0.out, rtol=1e-13, atol=1e-15)


def test_batch_independence():
    _, layer = tiny_seeded(seed=11)
    X = make_x(9, 32, seed=11, x_seed=4)
    whole = moe_forward(layer, X)
    for t in (0, 4, 8):
        alone = moe_forward(layer, X[t:t + 1])[0]
        np.testing.assert_array_equal(alone.out, whole[t].out)
        assert alone.ids.tolist() == whole[t].ids.tolist()


def test_linear_in_all_down_projections():
    """Scaling every W2 (routed and shared) by 2 scales the output by 2."""
    syn, layer = tiny_seeded(seed=13)
    two = lambda e: (syn.expert(e)[0],
                     f32_to_bf16_bits(2 * bf16_to_f64(syn.expert(e)[1]).astype(np.float32)))
    l2 = OracleLayer(32, 8, 3, 16, layer.router_w_bits, None, two)
    X = make_x(3, 32, seed=13, x_seed=5)
    for r1, r2 in zip(moe_forward(layer, X), moe_forward(l2, X)):
        np.testing.assert_allclose(r2.out, 2 * r1.out, rtol=1e-13, atol=1e-15)


def test_dense_special_case_k_equals_E_without_renorm():
    """k = E and renormalisation off: the layer is the dense sigmoid-gated
    mixture sum_e sigma(z_e) E_e(x) + shared(x), evaluated here densely."""
    syn, base = tiny_seeded(seed=17, E=8, k=8)
    X = make_x(3, 32, seed=17, x_seed=6)
    Wr = bf16_to_f64(syn.router_w()).reshape(8, 32)
    for t, r in enumerate(moe_forward(base, X, renormalize=False)):
        x = bf16_to_f64(X[t])
        acc = np.zeros(32)
        for e in list(range(8)) + [-1]:
            w13, w2 = syn.expert(e)
            y, _ = expert_forward(bf16_to_f64(w13).reshape(32, 32),
                                  bf16_to_f64(w2).reshape(32, 16), x, 16)
            gate = 1.0 if e < 0 else 1.0 / (1.0 + math.exp(-float(Wr[e] @ x)))
            acc += gate * y
        np.testing.assert_allclose(r.out, acc, rtol=1e-12, atol=1e-14)


def test_route_all_matches_per_token():
    _, layer = tiny_seeded(seed=19, with_bias=True)
    X = make_x(6, 32, seed=19, x_seed=7)
    ids, w, gaps, logits = route_all(layer, X)
    for t, r in enumerate(moe_forward(layer, X)):
        assert ids[t].tolist() == r.ids.tolist()
        np.testing.assert_array_equal(w[t], r.weights)
        assert gaps[t] == r.gap


# ---------------------------------------------------------------- bucketing

@pytest.mark.parametrize("T,E,k", [(1, 256, 6), (8, 256, 6), (33, 16, 4), (200, 8, 2)])
def test_bucket_invariants(T, E, k):
    rng = np.random.default_rng(T * 31 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    b = bucket(ids, E)
    flat = ids.reshape(-1)
    assert b["counts"].sum() == T * k
    assert b["offsets"][0] == 0 and b["offsets"][-1] == T * k
    assert np.all(np.diff(b["offsets"]) == b["counts"])
    assert sorted(b["slots"].tolist()) == list(range(T * k))      # a permutation
    assert b["active"].tolist() == sorted(set(flat.tolist()))     # the union, ascending
    for e in range(E):
        seg = b["slots"][b["offsets"][e]:b["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    if T == 1:
        assert sorted(b["active"].tolist()) == sorted(ids[0].tolist())

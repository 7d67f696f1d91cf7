"""Pins of the dense-MLP oracle (layers 0 and 1).

A wrong gate/up split of w13, a transposed w2, a missing SiLU or a dropped
residual each fail one of these.
"""

import math

import numpy as np

from oracle import OracleLayer, bf16_to_f64, moe_token
from oracle.dense import DenseMLP, mlp_block_forward, mlp_forward, mlp_token
from synth import SyntheticDenseMLP, f32_to_bf16_bits, make_x


def bits(a):
    a = np.asarray(a, dtype=np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_to_f64(b), a.astype(np.float64)), "value not bf16-exact"
    return b


def test_worked_example():
    # x = (1, 2); the gate row picks x0, the up row picks x1; w2 = (3, 0.5)^T.
    # h = silu(1) * 2 = 2 / (1 + e^-1) = 1.4621171572600098
    m = DenseMLP(2, 1, bits([[1.0, 0.0], [0.0, 1.0]]), bits([[3.0], [0.5]]))
    out, h = mlp_forward(m, bits([[1.0, 2.0]]))[0]
    np.testing.assert_allclose(h, [1.4621171572600098], rtol=1e-15)
    np.testing.assert_allclose(out, [4.386351471780029, 0.7310585786300049], rtol=1e-15)


def test_structured_rows_closed_form():
    """Gate row c reads x[a_c], up row c reads x[b_c], w2 column c writes
    output o_c: out[o_c] = silu(x[a_c]) * x[b_c] (distinct outputs)."""
    H, Id = 16, 5
    a, b, o = [3, 0, 7, 7, 12], [1, 9, 2, 15, 4], [0, 5, 6, 10, 11]
    w13 = np.zeros((2 * Id, H)); w2 = np.zeros((H, Id))
    for c in range(Id):
        w13[c, a[c]] = 1.0
        w13[Id + c, b[c]] = 1.0
        w2[o[c], c] = 1.0
    x = np.arange(H) / 4.0 - 1.75
    m = DenseMLP(H, Id, bits(w13), bits(w2))
    out, _ = mlp_forward(m, bits([x]))[0]
    want = np.zeros(H)
    for c in range(Id):
        xa = x[a[c]]
        want[o[c]] = xa / (1 + math.exp(-xa)) * x[b[c]]
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-15)


def test_intermediate_channels_add_up():
    """An MLP of width 2m is the sum of the two MLPs of width m made of its
    first and second halves of channels (gate, up and down sliced alike)."""
    S = SyntheticDenseMLP(seed=3, inter=96, hidden=64)
    w13, w2 = S.w13(), S.w2()
    m = 48
    full = DenseMLP(64, 96, w13, w2)
    lo = DenseMLP(64, m, np.concatenate([w13[:m], w13[96:96 + m]]), np.ascontiguousarray(w2[:, :m]))
    hi = DenseMLP(64, m, np.concatenate([w13[m:96], w13[96 + m:]]), np.ascontiguousarray(w2[:, m:]))
    X = make_x(3, hidden=64, seed=3, x_seed=0)
    for (yf, _), (yl, _), (yh, _) in zip(mlp_forward(full, X), mlp_forward(lo, X), mlp_forward(hi, X)):
        np.testing.assert_allclose(yf, yl + yh, rtol=1e-12, atol=1e-14)


def test_width_512_is_the_shared_expert_alone():
    """The layer with routed_scale 0 is its shared expert: an MLP with those
    weights gives the same output."""
    S = SyntheticDenseMLP(seed=5, inter=512, hidden=256)
    w13, w2 = S.w13(), S.w2()
    rng = np.random.default_rng(0)
    routed = {e: (f32_to_bf16_bits(rng.standard_normal((1024, 256)).astype(np.float32) * 0.02),
                  f32_to_bf16_bits(rng.standard_normal((256, 512)).astype(np.float32) * 0.02))
              for e in range(8)}
    L = OracleLayer(hidden=256, n_experts=8, top_k=2, inter=512,
                    router_w_bits=f32_to_bf16_bits(rng.standard_normal((8, 256)).astype(np.float32)),
                    router_b=None, expert_raw=lambda e: (w13, w2) if e < 0 else routed[e])
    X = make_x(2, hidden=256, seed=5, x_seed=1)
    mlp = DenseMLP(256, 512, w13, w2)
    for t, (y, _) in enumerate(mlp_forward(mlp, X)):
        np.testing.assert_allclose(y, moe_token(L, X[t], routed_scale=0.0).out, rtol=1e-13, atol=1e-15)


def test_block_zero_gamma_and_unit_rms():
    S = SyntheticDenseMLP(seed=7, inter=64, hidden=128)
    m = DenseMLP(128, 64, S.w13(), S.w2())
    R = make_x(2, hidden=128, seed=7, x_seed=2)
    for t, res in enumerate(mlp_block_forward(m, R, np.zeros(128, np.uint16))):
        np.testing.assert_array_equal(res.out, bf16_to_f64(R[t]))
    rng = np.random.default_rng(1)
    r = bits([np.where(rng.random(128) < 0.5, -1.0, 1.0)])
    res = mlp_block_forward(m, r, bits(np.ones(128)), eps=0.0)[0]
    assert np.array_equal(res.normed_bits, r[0])
    y, _ = mlp_token(*m.f64(), bf16_to_f64(r[0]), 64)
    np.testing.assert_array_equal(res.out, bf16_to_f64(r[0]) + y)

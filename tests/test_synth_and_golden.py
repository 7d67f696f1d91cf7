"""Input generator sanity and the oracle regression fixture."""

import json
import os

import numpy as np

from oracle import moe_forward
from synth import (LayerShape, SyntheticLayer, bf16_bits_to_f32, f32_to_bf16_bits, make_x)

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5], dtype=np.float32)
    b = f32_to_bf16_bits(f)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 (odd) and 1+2^-6 (even): rounds up.
    assert b.tolist()[:5] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    assert np.array_equal(bf16_bits_to_f32(b)[[0, 4]], np.float32([1.0, -2.5]))


def test_streams_are_per_tensor_and_deterministic():
    shp = LayerShape(hidden=64, n_experts=6, top_k=2, inter=16)
    a, b = SyntheticLayer(4, shp), SyntheticLayer(4, shp)
    w13, w2 = a.routed_banks(threads=3)
    assert np.array_equal(w13[3], b.w13(3)) and np.array_equal(w2[5], b.w2(5))
    assert not np.array_equal(a.w13(0), a.w13(1))
    assert np.array_equal(make_x(3, 64, seed=4), make_x(3, 64, seed=4))
    assert not np.array_equal(make_x(3, 64, seed=4, x_seed=1), make_x(3, 64, seed=4))


def test_distributions():
    syn = SyntheticLayer(0)
    w = bf16_bits_to_f32(syn.w13(0)).astype(np.float64)
    assert abs(w.std() - 0.02) < 2e-4 and abs(w.mean()) < 1e-4
    x = bf16_bits_to_f32(make_x(64)).astype(np.float64)
    assert abs(x.std() - 1.0) < 0.02
    b = syn.router_bias()
    assert b.shape == (256,) and b.dtype == np.float32


def test_oracle_regression_fixture():
    """Written by tests/golden/make_golden.py from the oracle alone."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(HERE, "golden", "oracle_tiny_seed7.json")) as f:
        doc = json.load(f)
    layer, x = mg.build()
    res = moe_forward(layer, x)
    for t, r in enumerate(res):
        assert r.ids.tolist() == doc["ids"][t]
        np.testing.assert_allclose(r.weights, doc["weights"][t], rtol=1e-14)
        np.testing.assert_allclose(r.gap, doc["gaps"][t], rtol=1e-12)
        np.testing.assert_allclose(r.out, doc["out"][t], rtol=1e-12, atol=1e-15)

"""Pins of the oracle's NVFP4 decoding (format tables, layout) and of the
synthetic NVFP4 encoder's round trip."""

import numpy as np
import pytest
import torch

from oracle import OracleLayer, bf16_to_f64, e2m1_to_f64, e4m3fn_to_f64, moe_forward, nvfp4_dequant
from synth import LayerShape, SyntheticLayer, f32_to_bf16_bits, make_x, quantize_nvfp4


def test_e2m1_codes_against_format_formula():
    """OCP MX v1.0 FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
    exponent 0 is subnormal (0.5 * m)."""
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        v = (0.5 * m) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        v = -v if s else v
        assert e2m1_to_f64(np.array([code]))[0] == v, code


def test_e4m3fn_all_bytes_against_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_to_f64(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert e4m3fn_to_f64(np.array([0x7E]))[0] == 448.0
    assert e4m3fn_to_f64(np.array([0x01]))[0] == 2.0 ** -9


def test_dequant_nibble_order_and_block_index():
    """Hand-built row of K = 48: byte j holds k = 2j in its low nibble; block
    b = k // 16 uses scale byte b."""
    K = 48
    codes = np.array([(3 * k + 1) % 16 for k in range(K)], dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0x38, 0x40, 0x30]], dtype=np.uint8)   # 1.0, 2.0, 0.5
    g = 0.125
    w = nvfp4_dequant(packed, scales, g)[0]
    table = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for k in range(K):
        c = int(codes[k])
        v = (-1 if c & 8 else 1) * table[c & 7] * [1.0, 2.0, 0.5][k // 16] * g
        assert w[k] == v, k


def test_quantizer_round_trip_of_representable_values():
    """Values already of the form e2m1 * e4m3 * g come back exactly."""
    rng = np.random.default_rng(0)
    rows, K = 4, 64
    g = 2.0 ** -10
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    q = rng.choice(table, size=(rows, K)) * rng.choice([-1, 1], size=(rows, K))
    q[:, ::16] = 6.0                     # every block reaches the top code
    s = 2.0 ** rng.integers(-3, 4, size=(rows, K // 16))
    w = q * np.repeat(s, 16, axis=1) * g * (6 * 448) / 6  # choose g_tensor = amax/(6*448)
    wb = f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_to_f64(wb), w)
    t = quantize_nvfp4(wb)
    np.testing.assert_array_equal(nvfp4_dequant(t.packed, t.scales, t.gscale), w)


def test_quantizer_error_is_bounded():
    """Per-element error of the synthetic encoder is at most half an E2M1 step
    of its block (plus the E4M3 scale rounding) — a sanity bound, not parity."""
    syn = SyntheticLayer(0, LayerShape(hidden=256, n_experts=2, top_k=1, inter=64))
    wb = syn.w13(0)
    t = quantize_nvfp4(wb)
    w = bf16_to_f64(wb)
    d = nvfp4_dequant(t.packed, t.scales, t.gscale)
    rel = np.sqrt(np.mean((d - w) ** 2) / np.mean(w ** 2))
    assert rel < 0.15
    assert np.max(np.abs(d)) <= np.max(np.abs(w)) * (1 + 1 / 8)


def test_nvfp4_layer_equals_bf16_layer_on_decoded_weights():
    """The NVFP4 oracle is the bf16 oracle on the decoded weights.  With a
    power-of-two tensor scale every decoded value (<= 2 + 4 significant bits)
    is bf16-exact, so the two layers must agree bit for bit."""
    shp = LayerShape(hidden=64, n_experts=8, top_k=2, inter=32)
    syn = SyntheticLayer(21, shp)
    g = np.float32(2.0 ** -12)
    q = {}
    for e in list(range(8)) + [-1]:
        a, b = (quantize_nvfp4(syn.expert(e)[i]) for i in (0, 1))
        q[e] = ((a.packed, a.scales, g), (b.packed, b.scales, g))

    def raw16(e):
        return tuple(f32_to_bf16_bits(nvfp4_dequant(*q[e][i]).astype(np.float32)) for i in (0, 1))

    for e in q:
        for i in (0, 1):
            assert np.array_equal(bf16_to_f64(raw16(e)[i]), nvfp4_dequant(*q[e][i]))
    l4 = OracleLayer(64, 8, 2, 32, syn.router_w(), None, lambda e: q[e], fmt="nvfp4")
    l16 = OracleLayer(64, 8, 2, 32, syn.router_w(), None, raw16)
    X = make_x(3, 64, seed=21)
    for a, b in zip(moe_forward(l4, X), moe_forward(l16, X)):
        np.testing.assert_array_equal(a.out, b.out)

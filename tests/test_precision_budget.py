"""Precision budget of the prefill path's intermediate formats, on the CPU.

The prefill GEMMs keep h as fp16 between the gate/up and down products and
store each slot's unweighted down projection y as fp16 for the combine, both
with a power-of-two bias (h is stored as fp16(h * 2^-8), so y comes out of
the down GEMM as y * 2^-8; the combine multiplies by 2^8); the output is
rounded once to bf16.  This test replays those roundings in NumPy on top of
the fp64 oracle's own h and weights, for a spread sample of the T = 8192
prefill workload's tokens, and checks that the result stays inside the
layer's tolerance (2e-2 x RMS of the oracle output), that the fp16
intermediates alone add at most a tenth of it, and that a single bf16
rounding of h, the obvious alternative, costs several times more.  A second
case scales every gate/up weight by 2^8, which pushes |h| and |y| far past
fp16's 65504: unbiased fp16 overflows there, the biased form stays inside
the tolerance.
"""

import numpy as np
import pytest

from oracle import OracleLayer, bf16_to_f64, moe_forward
from oracle.block import f64_to_bf16_bits
from oracle.grading import TOL_BF16
from synth import LayerShape, SyntheticLayer, make_x

N_SAMPLE = 32
# The scaled-weight case drives the SiLU into exp overflow (-> 0, its limit).
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f16(v):
    return v.astype(np.float16).astype(np.float64)


def _f16_biased(v):
    """fp16 storage of v * 2^-8, read back and multiplied by 2^8."""
    with np.errstate(over="ignore"):
        return (v * 2.0 ** -8).astype(np.float16).astype(np.float64) * 2.0 ** 8


def _bf16(v):
    return bf16_to_f64(f64_to_bf16_bits(v))


def _replayer(L, res):
    cache = {}

    def w2(e):
        if e not in cache:
            cache[e] = L.expert_f64(e)[1]
        return cache[e]

    def replay(h_round, y_round, out_round):
        err = []
        for r in res:
            # The shared GEMM's y stays in the fp32 accumulator.
            out = w2(-1) @ h_round(r.h_shared)
            for j, e in enumerate(r.ids):
                out = out + r.weights[j] * y_round(w2(int(e)) @ h_round(r.h_routed[j]))
            err.append(out_round(out) - r.out)
        rms = np.sqrt(np.mean(np.stack([r.out for r in res]) ** 2))
        return float(np.max(np.abs(err)) / rms)

    return replay


def test_prefill_intermediate_roundings_fit_the_tolerance():
    S = SyntheticLayer(0)
    L = OracleLayer(2048, 256, 6, 512, S.router_w(), None, S.expert)
    T = 8192
    X = make_x(T, seed=0, x_seed=0)
    toks = np.linspace(0, T - 1, N_SAMPLE).astype(int).tolist()
    replay = _replayer(L, moe_forward(L, X, tokens=toks))
    used = replay(_f16_biased, _f16_biased, _bf16)    # the formats the prefill kernels use
    no_out = replay(_f16_biased, _f16_biased, lambda v: v)   # without the final bf16 rounding
    plain = replay(_f16, _f16, lambda v: v)           # unbiased fp16: the same here
    bf16_h = replay(_bf16, lambda v: v, lambda v: v)
    print(f"biased fp16 h + y + bf16 out: {used:.4f}; before the output rounding: {no_out:.4f} "
          f"(unbiased {plain:.4f}); bf16 h alone: {bf16_h:.4f} (tolerance {TOL_BF16})")
    # The output's own bf16 rounding takes most of the budget (up to 2^-9 |out|);
    # the intermediate formats add a tenth of the tolerance at most, and the
    # bias costs nothing at these magnitudes.
    assert used <= TOL_BF16
    assert no_out <= TOL_BF16 / 10
    assert no_out <= 1.05 * plain
    assert bf16_h >= 4 * no_out


def scaled_gateup_layer(S, factor=256.0, n_experts=16):
    """The seeded layer with every gate/up weight (routed and shared) times a
    power of two (exact in bf16): h grows by factor^2, y by factor^2."""
    from oracle.block import f64_to_bf16_bits as to_bits

    def raw(e):
        w13, w2 = S.expert(e)
        return to_bits(bf16_to_f64(w13) * factor).reshape(w13.shape), w2

    return OracleLayer(2048, n_experts, 6, 512, S.router_w(), None, raw)


def test_prefill_biased_fp16_keeps_large_activations():
    S = SyntheticLayer(3, LayerShape(n_experts=16))
    L = scaled_gateup_layer(S)
    X = make_x(300, seed=3, x_seed=1)
    res = moe_forward(L, X, tokens=list(range(0, 300, 10)))
    h_max = max(max(np.max(np.abs(r.h_routed)), np.max(np.abs(r.h_shared))) for r in res)
    assert h_max > 4 * 65504, h_max
    replay = _replayer(L, res)
    with np.errstate(over="ignore", invalid="ignore"):
        plain = replay(_f16, _f16, _bf16)
    used = replay(_f16_biased, _f16_biased, _bf16)
    print(f"max |h| {h_max:.3e}: unbiased fp16 {plain}, biased fp16 {used:.4f} (tolerance {TOL_BF16})")
    assert not np.isfinite(plain)
    assert used <= TOL_BF16


def test_nvfp4_decode_bf16_h_fits_the_tolerance():
    """W4A16 (NVFP4 weights, 16-bit activations): the decode kernels round h
    once to bf16 between the two GEMVs.  Replayed on the fp64 oracle's h of
    32 tokens of a 16-expert NVFP4 layer, that rounding alone stays under a
    quarter of the NVFP4 tolerance (5e-2 x RMS), and with the bf16 output
    rounding the total stays under a third of it."""
    from oracle.grading import TOL_NVFP4
    from synth.nvfp4_pack import quantize_nvfp4
    S = SyntheticLayer(5, LayerShape(n_experts=16))
    cache = {}

    def raw(e):
        if e not in cache:
            w13, w2 = S.expert(e)
            a, b = quantize_nvfp4(w13), quantize_nvfp4(w2)
            cache[e] = ((a.packed, a.scales, a.gscale), (b.packed, b.scales, b.gscale))
        return cache[e]

    L = OracleLayer(2048, 16, 6, 512, S.router_w(), None, raw, fmt="nvfp4")
    res = moe_forward(L, make_x(32, seed=5, x_seed=2))
    replay = _replayer(L, res)
    used = replay(_bf16, lambda v: v, _bf16)          # bf16 h, fp32 y, bf16 output
    out_only = replay(lambda v: v, lambda v: v, _bf16)
    no_out = replay(_bf16, lambda v: v, lambda v: v)   # bf16 h, output unrounded
    print(f"NVFP4 decode: bf16 h + bf16 out {used:.5f}; bf16 out alone {out_only:.5f}; "
          f"bf16 h alone {no_out:.5f} (tolerance {TOL_NVFP4})")
    # Measured: 0.0134 with both roundings (the output's own rounding alone
    # gives the same worst element), 0.0088 from the bf16 h alone -- too much
    # for the bf16 layer's 2e-2 budget, which is why h stays fp32 there.
    assert used <= TOL_NVFP4 / 3
    assert no_out <= TOL_NVFP4 / 4

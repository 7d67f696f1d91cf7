"""Precision budget of the prefill path's intermediate formats, on the CPU.

The prefill GEMMs keep h as fp16 between the gate/up and down products and
store each slot's unweighted down projection y as fp16 for the combine; the
output is rounded once to bf16.  This test replays those roundings in NumPy
on top of the fp64 oracle's own h and weights, for a spread sample of the
T = 8192 prefill workload's tokens, and checks that the result stays inside
the layer's tolerance (2e-2 x RMS of the oracle output), that the fp16
intermediates alone add at most a tenth of it, and that a single bf16
rounding of h, the obvious alternative, costs several times more.
"""

import numpy as np

from oracle import OracleLayer, bf16_to_f64, moe_forward
from oracle.block import f64_to_bf16_bits
from oracle.grading import TOL_BF16
from synth import SyntheticLayer, make_x

N_SAMPLE = 32


def _f16(v):
    return v.astype(np.float16).astype(np.float64)


def _bf16(v):
    return bf16_to_f64(f64_to_bf16_bits(v))


def test_prefill_intermediate_roundings_fit_the_tolerance():
    S = SyntheticLayer(0)
    L = OracleLayer(2048, 256, 6, 512, S.router_w(), None, S.expert)
    T = 8192
    X = make_x(T, seed=0, x_seed=0)
    toks = np.linspace(0, T - 1, N_SAMPLE).astype(int).tolist()
    res = moe_forward(L, X, tokens=toks)
    cache = {}

    def w2(e):
        if e not in cache:
            cache[e] = L.expert_f64(e)[1]
        return cache[e]

    def replay(h_round, y_round, out_round):
        err = []
        for r in res:
            out = w2(-1) @ h_round(r.h_shared)          # the shared GEMM's y stays fp32
            for j, e in enumerate(r.ids):
                out = out + r.weights[j] * y_round(w2(int(e)) @ h_round(r.h_routed[j]))
            err.append(out_round(out) - r.out)
        rms = np.sqrt(np.mean(np.stack([r.out for r in res]) ** 2))
        return float(np.max(np.abs(err)) / rms)

    used = replay(_f16, _f16, _bf16)            # the formats the prefill kernels use
    no_out = replay(_f16, _f16, lambda v: v)    # the same without the final bf16 rounding
    bf16_h = replay(_bf16, lambda v: v, lambda v: v)
    print(f"fp16 h + fp16 y + bf16 out: {used:.4f}; before the output rounding: {no_out:.4f}; "
          f"bf16 h alone: {bf16_h:.4f} (tolerance {TOL_BF16})")
    # The output's own bf16 rounding takes most of the budget (up to 2^-9 |out|);
    # the intermediate formats add a tenth of the tolerance at most.
    assert used <= TOL_BF16
    assert no_out <= TOL_BF16 / 10
    assert bf16_h >= 4 * no_out

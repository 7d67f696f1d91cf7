"""Write the oracle regression fixture ``oracle_tiny_seed7.json``.

Calls only ``oracle/`` (and ``synth/`` for the seeded inputs).  The fixture
freezes the oracle's output on a small seeded layer so that any later change
to the oracle's arithmetic shows up as a failing test and has to be justified.

    python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import OracleLayer, moe_forward  # noqa: E402
from synth import LayerShape, SyntheticLayer, make_x  # noqa: E402

SHAPE = dict(hidden=64, n_experts=16, top_k=4, inter=32)
SEED, T, X_SEED = 7, 5, 0


def build():
    syn = SyntheticLayer(SEED, LayerShape(**SHAPE))
    layer = OracleLayer(router_w_bits=syn.router_w(), router_b=syn.router_bias(),
                        expert_raw=syn.expert, **SHAPE)
    x = make_x(T, SHAPE["hidden"], seed=SEED, x_seed=X_SEED)
    return layer, x


def main():
    layer, x = build()
    res = moe_forward(layer, x)
    doc = {
        "what": "oracle output of a seeded tiny layer (router bias on, renormalize on)",
        "shape": SHAPE, "seed": SEED, "T": T, "x_seed": X_SEED,
        "ids": [r.ids.tolist() for r in res],
        "weights": [r.weights.tolist() for r in res],
        "gaps": [r.gap for r in res],
        "out": [r.out.tolist() for r in res],
    }
    with open(os.path.join(HERE, "oracle_tiny_seed7.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()

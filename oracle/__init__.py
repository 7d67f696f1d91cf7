"""CPU oracle for the Flint MoE feed-forward layer — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, fp64 reference that the HIP path is graded
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path
(``sparse_expert_gemv_amd``) never imports, links or calls anything here, and
this package never imports the product path: the two share no code.  The only
module both sides use is ``synth`` (seeded input generation, no layer
arithmetic).

Pins (tests marked ``not gpu`` in ``tests/test_oracle_*.py``): every function
below is checked against something other than itself — closed forms, brute
force over all subsets on tiny inputs, structured weights whose output has a
closed form, invariants of the layer (shared-expert-only output, permutation
equivariance, batch independence, linearity), special cases that reduce to a
dense mixture, and the FP8/FP4 code tables of the format definitions.  The
pre-norm block (``block``) is pinned by a worked example, closed forms of the
norm, every bf16 rounding midpoint, and reductions to the residual alone and to
the bare layer.  The dense MLP of layers 0 and 1 (``dense``) is pinned by a
worked example, structured rows with a closed form, additivity over
intermediate channels, and its reduction to the layer's shared expert.  The
low-latency decode path around the layer (``decoder``: attention output
projection, rounded residual adds, the next layer's norm) is pinned by a
brute-force projection, hand-worked residual roundings, closed forms of the
next norm, and its reduction to the block oracle when the projection is
zero.  The expert-grouped evaluation (``grouped``) is pinned token by token
against the per-token oracle.

Parity unpinned: agreement with Recursive's own runtime at the real Flint
shape cannot be checked here (neither that runtime nor trained weights are
available); the pages print no worked numeric example of the layer.
"""

from .moe import (  # noqa: F401
    OracleLayer,
    TokenResult,
    bf16_to_f64,
    router_logits,
    sigmoid,
    silu,
    select_topk,
    routing_weights,
    expert_forward,
    moe_token,
    moe_forward,
    bucket,
    route_all,
)
from .block import BlockResult, block_forward, block_token, f64_to_bf16_bits, rmsnorm  # noqa: F401
from .dense import DenseMLP, mlp_block_forward, mlp_forward, mlp_token  # noqa: F401
from .decoder import DecoderResult, decoder_forward, decoder_token, o_proj  # noqa: F401
from .nvfp4 import e2m1_to_f64, e4m3fn_to_f64, nvfp4_dequant  # noqa: F401

"""Seeded synthetic inputs for the Flint MoE feed-forward layer.

This package only *produces inputs* (weights, activations, router bias and the
NVFP4 byte encoding of the weights).  It holds none of the layer's arithmetic:
both the CPU oracle (``oracle/``) and the HIP path consume what it returns, and
neither imports the other.
"""

from .flint_layer import (  # noqa: F401
    FLINT_HIDDEN,
    FLINT_N_EXPERTS,
    FLINT_TOP_K,
    FLINT_INTER,
    LayerShape,
    SyntheticLayer,
    SyntheticDenseMLP,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    make_x,
    make_residual,
    make_o_proj,
    make_attn,
    make_next_gain,
)
from .nvfp4_pack import quantize_nvfp4, NvFp4Tensor  # noqa: F401

"""MI355X (gfx950) Flint MoE feed-forward layer: HIP kernels behind a C ABI.

``libflint_moe.so`` (built from ``csrc/`` by ``build.py``) holds the router
GEMV with sigmoid top-k, the token-to-expert bucketing, the fused gate/up GEMV
with SiLU-and-mul, and the down GEMV with the routing-weight combine; the
pre-norm block around the layer (RMSNorm + residual add); and the dense
SwiGLU MLP of Flint's first two layers.
``flint_moe`` is the ctypes binding; it raises if the library is missing.
"""

from .flint_moe import (  # noqa: F401
    FLINT_OK, FLINT_ERR_INVALID_ARG, FLINT_ERR_UNSUPPORTED, FLINT_ERR_WORKSPACE, FLINT_ERR_HIP,
    FLINT_W_BF16, FLINT_W_NVFP4, ABI_SYMBOLS, LIB_PATH, DeviceBank, DeviceWeights, FlintError,
    FlintMoE, FlintMLP, CALIB_SINK_WORDS, bf16_bits, bf16_tensor, calib_stream_read, load_library,
    status_string,
)

"""NVFP4 decoding for the oracle (fp64) — test infrastructure only.

The pages say the NVFP4 checkpoint runs weight-only (W4A16) with bf16
activations ("vLLM Day-0 Support for Recursive's Flint", section "Flint Model
Overview and Capabilities"; "RecursiveSI/flint — vLLM serving recipe", section
"Guide / Overview").  They do not print the byte layout.  Reading used here
(and by the kernels, which do not share this code):

  W[r, k] = e2m1(nibble(r, k)) * e4m3fn(scale[r, k // 16]) * g

with the even k in the low nibble of byte k // 2, nibble bit 3 the sign.

Pins: every E2M1 code against the sign/exponent/mantissa formula of the OCP
Microscaling (MX) v1.0 FP4 definition; all 256 E4M3FN bytes against PyTorch's
``float8_e4m3fn`` conversion; a hand-built row for nibble order and block
indexing (``tests/test_oracle_nvfp4.py``).
"""

from __future__ import annotations

import numpy as np

# E2M1 magnitudes indexed by the low three bits of a code.
_E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (0..15) to fp64: bit 3 sign, bits 2..0 magnitude index."""
    c = np.asarray(codes).astype(np.int64)
    mag = _E2M1_MAGNITUDE[c & 7]
    return np.where(c & 8, -mag, mag)


def e4m3fn_to_f64(b: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN bytes to fp64: bias 7, subnormals at exponent 0, NaN at 0x7F/0xFF."""
    b = np.asarray(b).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((b & 0x7F) == 0x7F, np.nan, v)


def nvfp4_dequant(packed: np.ndarray, scales: np.ndarray, gscale: float) -> np.ndarray:
    """Decode one NVFP4 matrix: packed uint8 [rows, K/2], scales uint8 [rows, K/16]."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    K = 2 * half
    codes = np.empty((rows, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    q = e2m1_to_f64(codes)
    s = e4m3fn_to_f64(scales)
    s_per_k = np.repeat(s, 16, axis=1)
    return q * s_per_k * float(gscale)

"""Copy a synthetic layer's tensors to GPU memory (PyTorch tensors).

Returns plain tensors keyed by name; the product binding wraps them into the
structures its C ABI takes.  bf16 tensors are uploaded bit-exactly as
``torch.bfloat16``; NVFP4 tensors as ``torch.uint8`` bytes and fp32 scales.
"""

from __future__ import annotations

import numpy as np
import torch

from .flint_layer import SyntheticLayer
from .nvfp4_pack import quantize_nvfp4


def _bf16(bits: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def upload_bf16(syn: SyntheticLayer, device="cuda", with_bias: bool = False) -> dict:
    w13, w2 = syn.routed_banks()
    sw13, sw2 = syn.shared()
    return {
        "router_w": _bf16(syn.router_w(), device),
        "router_b": torch.from_numpy(syn.router_bias().copy()).to(device) if with_bias else None,
        "w13": _bf16(w13, device), "w2": _bf16(w2, device),
        "sh_w13": _bf16(sw13[None], device), "sh_w2": _bf16(sw2[None], device),
    }


def nvfp4_layer(syn: SyntheticLayer, threads: int = 8) -> dict:
    """NVFP4 encoding of every routed expert and the shared expert (host arrays).

    Keys: for bank in (routed, shared): w13_q / w13_s / w13_g and w2_q / w2_s /
    w2_g (packed codes, E4M3 block scales, fp32 tensor scale), stacked on a
    leading expert axis."""
    from concurrent.futures import ThreadPoolExecutor
    E = syn.shape.n_experts
    out = {}
    for name, ids in (("routed", list(range(E))), ("shared", [-1])):
        def enc(e):
            a, b = syn.expert(e)
            return quantize_nvfp4(a), quantize_nvfp4(b)
        with ThreadPoolExecutor(max_workers=threads) as ex:
            encs = list(ex.map(enc, ids))
        out[name] = {
            "w13_q": np.stack([qa.packed for qa, _ in encs]),
            "w13_s": np.stack([qa.scales for qa, _ in encs]),
            "w13_g": np.array([qa.gscale for qa, _ in encs], dtype=np.float32),
            "w2_q": np.stack([qb.packed for _, qb in encs]),
            "w2_s": np.stack([qb.scales for _, qb in encs]),
            "w2_g": np.array([qb.gscale for _, qb in encs], dtype=np.float32),
        }
    return out


def upload_nvfp4(syn: SyntheticLayer, q: dict, device="cuda", with_bias: bool = False) -> dict:
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    d = {"router_w": _bf16(syn.router_w(), device),
         "router_b": torch.from_numpy(syn.router_bias().copy()).to(device) if with_bias else None}
    for name in ("routed", "shared"):
        for k, v in q[name].items():
            d[f"{name}_{k}"] = t(v)
    return d

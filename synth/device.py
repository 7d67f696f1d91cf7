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


def nvfp4_layer(syn: SyntheticLayer) -> dict:
    """NVFP4 encoding of every routed expert and the shared expert (host arrays).

    Keys: for bank in (routed, shared): packed/scale/gscale of w13 and w2,
    stacked on a leading expert axis."""
    E = syn.shape.n_experts
    out = {}
    for name, ids in (("routed", list(range(E))), ("shared", [-1])):
        parts = {k: [] for k in ("w13_q", "w13_s", "w13_g", "w2_q", "w2_s", "w2_g")}
        for e in ids:
            a, b = syn.expert(e)
            qa, qb = quantize_nvfp4(a), quantize_nvfp4(b)
            parts["w13_q"].append(qa.packed); parts["w13_s"].append(qa.scales); parts["w13_g"].append(qa.gscale)
            parts["w2_q"].append(qb.packed); parts["w2_s"].append(qb.scales); parts["w2_g"].append(qb.gscale)
        out[name] = {k: (np.stack(v) if k[-1] != "g" else np.array(v, dtype=np.float32))
                     for k, v in parts.items()}
    return out


def upload_nvfp4(syn: SyntheticLayer, q: dict, device="cuda", with_bias: bool = False) -> dict:
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    d = {"router_w": _bf16(syn.router_w(), device),
         "router_b": torch.from_numpy(syn.router_bias().copy()).to(device) if with_bias else None}
    for name in ("routed", "shared"):
        for k, v in q[name].items():
            d[f"{name}_{k}"] = t(v)
    return d

"""ctypes binding of ``libflint_moe.so`` (argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
``include/flint_moe.h``; this module only converts PyTorch tensors into the
pointers and sizes that ABI takes.  PyTorch provides device memory and the
current stream.  There is no fallback: if the library is missing, loading it
raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflint_moe.so")

FLINT_OK = 0
FLINT_ERR_INVALID_ARG = 1
FLINT_ERR_UNSUPPORTED = 2
FLINT_ERR_WORKSPACE = 3
FLINT_ERR_HIP = 4

FLINT_W_BF16 = 0
FLINT_W_NVFP4 = 1

HEADER_BYTES = 21504  # FLINT_MOE_WS_HEADER_BYTES

# Symbols the header declares; tests check the library exports each of them.
ABI_SYMBOLS = (
    "flint_moe_init",
    "flint_moe_workspace_bytes",
    "flint_moe_workspace_layout",
    "flint_moe_forward",
    "flint_moe_forward_timed",
    "flint_moe_forward_noalloc",
    "flint_moe_block_forward",
    "flint_moe_block_forward_timed",
    "flint_moe_lowlat_forward",
    "flint_moe_lowlat_forward_timed",
    "flint_moe_destroy",
    "flint_moe_status_string",
    "flint_moe_last_error",
    "flint_mlp_init",
    "flint_mlp_workspace_bytes",
    "flint_mlp_workspace_layout",
    "flint_mlp_forward",
    "flint_mlp_forward_timed",
    "flint_mlp_destroy",
    "flint_mlp_last_error",
    "flint_moe_calib_stream_read",
)
CALIB_SINK_WORDS = 2048  # FLINT_MOE_CALIB_SINK_WORDS


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("format", ctypes.c_int32)]


class ExpertBank(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("w13_gscale", ctypes.c_void_p), ("w2_gscale", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("routed", ExpertBank), ("shared", ExpertBank)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("total_bytes", "header", "logits", "topk_ids", "topk_w",
                 "route", "h", "extra", "normed", "resid1", "norm_part", "items")]


class MlpConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32)]


class MlpWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("total_bytes", "normed", "h")]


class FlintError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m sparse_expert_gemv_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.flint_moe_init.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P)]
    lib.flint_moe_init.restype = ctypes.c_int
    lib.flint_moe_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.flint_moe_workspace_bytes.restype = ctypes.c_size_t
    lib.flint_moe_workspace_layout.argtypes = [P, ctypes.c_int32, ctypes.POINTER(WsLayout)]
    lib.flint_moe_workspace_layout.restype = ctypes.c_int
    lib.flint_moe_forward.argtypes = [P, ctypes.POINTER(Weights), P, ctypes.c_int32, P, P, P, P,
                                      ctypes.c_size_t, P]
    lib.flint_moe_forward.restype = ctypes.c_int
    lib.flint_moe_forward_timed.argtypes = [P, ctypes.POINTER(Weights), P, ctypes.c_int32, P, P, P,
                                            P, ctypes.c_size_t, P, ctypes.POINTER(P),
                                            ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.flint_moe_forward_timed.restype = ctypes.c_int
    lib.flint_moe_forward_noalloc.argtypes = [P, ctypes.POINTER(Weights), P, ctypes.c_int32, P, P,
                                              P, P]
    lib.flint_moe_forward_noalloc.restype = ctypes.c_int
    lib.flint_moe_block_forward.argtypes = [P, ctypes.POINTER(Weights), P, ctypes.c_float, P,
                                            ctypes.c_int32, P, P, P, P, ctypes.c_size_t, P]
    lib.flint_moe_block_forward.restype = ctypes.c_int
    lib.flint_moe_block_forward_timed.argtypes = [P, ctypes.POINTER(Weights), P, ctypes.c_float, P,
                                                  ctypes.c_int32, P, P, P, P, ctypes.c_size_t, P,
                                                  ctypes.POINTER(P), ctypes.c_int32,
                                                  ctypes.POINTER(ctypes.c_int32)]
    lib.flint_moe_block_forward_timed.restype = ctypes.c_int
    ll = [P, ctypes.POINTER(Weights), P, P, P, P, P, ctypes.c_float, ctypes.c_int32, P, P, P, P,
          P, ctypes.c_size_t, ctypes.c_int32, P]
    lib.flint_moe_lowlat_forward.argtypes = ll
    lib.flint_moe_lowlat_forward.restype = ctypes.c_int
    lib.flint_moe_lowlat_forward_timed.argtypes = ll + [ctypes.POINTER(P), ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_int32)]
    lib.flint_moe_lowlat_forward_timed.restype = ctypes.c_int
    lib.flint_mlp_init.argtypes = [ctypes.POINTER(MlpConfig), ctypes.POINTER(P)]
    lib.flint_mlp_init.restype = ctypes.c_int
    lib.flint_mlp_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.flint_mlp_workspace_bytes.restype = ctypes.c_size_t
    lib.flint_mlp_workspace_layout.argtypes = [P, ctypes.c_int32, ctypes.POINTER(MlpWsLayout)]
    lib.flint_mlp_workspace_layout.restype = ctypes.c_int
    lib.flint_mlp_forward.argtypes = [P, P, P, P, ctypes.c_float, P, ctypes.c_int32, P, P,
                                      ctypes.c_size_t, P]
    lib.flint_mlp_forward.restype = ctypes.c_int
    lib.flint_mlp_forward_timed.argtypes = [P, P, P, P, ctypes.c_float, P, ctypes.c_int32, P, P,
                                            ctypes.c_size_t, P, ctypes.POINTER(P), ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32)]
    lib.flint_mlp_forward_timed.restype = ctypes.c_int
    lib.flint_mlp_destroy.argtypes = [P]
    lib.flint_mlp_destroy.restype = None
    lib.flint_mlp_last_error.argtypes = [P]
    lib.flint_mlp_last_error.restype = ctypes.c_char_p
    lib.flint_moe_destroy.argtypes = [P]
    lib.flint_moe_destroy.restype = None
    lib.flint_moe_status_string.argtypes = [ctypes.c_int]
    lib.flint_moe_status_string.restype = ctypes.c_char_p
    lib.flint_moe_last_error.argtypes = [P]
    lib.flint_moe_last_error.restype = ctypes.c_char_p
    lib.flint_moe_calib_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.flint_moe_calib_stream_read.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().flint_moe_status_string(status).decode()


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None for None)."""
    return None if t is None else int(t.data_ptr())


@dataclass
class DeviceBank:
    """Tensors of one expert bank (bf16: w13, w2; NVFP4: + scales and gscales)."""
    w13: object
    w2: object
    w13_scale: object = None
    w2_scale: object = None
    w13_gscale: object = None
    w2_gscale: object = None

    def struct(self) -> ExpertBank:
        return ExpertBank(_ptr(self.w13), _ptr(self.w2), _ptr(self.w13_scale),
                          _ptr(self.w2_scale), _ptr(self.w13_gscale), _ptr(self.w2_gscale))


@dataclass
class DeviceWeights:
    router_w: object            # bf16 [E, H]
    router_b: object            # fp32 [E] or None
    routed: DeviceBank
    shared: DeviceBank

    def struct(self) -> Weights:
        return Weights(_ptr(self.router_w), _ptr(self.router_b), self.routed.struct(),
                       self.shared.struct())


class FlintMoE:
    """One layer configuration (a ``flint_moe_ctx``)."""

    def __init__(self, hidden=2048, n_experts=256, top_k=6, inter=512, max_tokens=64,
                 renormalize=True, routed_scale=1.0, fmt=FLINT_W_BF16):
        self.lib = load_library()
        self.cfg = Config(hidden, n_experts, top_k, inter, max_tokens, int(bool(renormalize)),
                          float(routed_scale), int(fmt))
        h = ctypes.c_void_p()
        st = self.lib.flint_moe_init(ctypes.byref(self.cfg), ctypes.byref(h))
        if st != FLINT_OK:
            raise FlintError(st, f"flint_moe_init: {status_string(st)}")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.flint_moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def top_k(self) -> int:
        return self.cfg.top_k

    def workspace_bytes(self, T: int) -> int:
        return int(self.lib.flint_moe_workspace_bytes(self.handle, T))

    def workspace_layout(self, T: int) -> dict:
        L = WsLayout()
        st = self.lib.flint_moe_workspace_layout(self.handle, T, ctypes.byref(L))
        if st != FLINT_OK:
            raise FlintError(st, f"flint_moe_workspace_layout: {status_string(st)}")
        return {n: getattr(L, n) for n, _ in WsLayout._fields_}

    def last_error(self) -> str:
        return self.lib.flint_moe_last_error(self.handle).decode()

    def forward_raw(self, weights: Weights, x_ptr, T, out_ptr, ids_ptr, w_ptr, ws_ptr, ws_bytes,
                    stream_ptr) -> int:
        """The C call with raw addresses; returns the status code."""
        return self.lib.flint_moe_forward(self.handle, ctypes.byref(weights), x_ptr, T, out_ptr,
                                          ids_ptr, w_ptr, ws_ptr, ws_bytes, stream_ptr)

    def forward_timed_raw(self, weights: Weights, x_ptr, T, out_ptr, ids_ptr, w_ptr, ws_ptr,
                          ws_bytes, stream_ptr, event_handles) -> tuple:
        """The timed C call; returns (status, number of kernels launched)."""
        n = len(event_handles)
        arr = (ctypes.c_void_p * n)(*event_handles)
        nk = ctypes.c_int32(0)
        st = self.lib.flint_moe_forward_timed(self.handle, ctypes.byref(weights), x_ptr, T, out_ptr,
                                              ids_ptr, w_ptr, ws_ptr, ws_bytes, stream_ptr, arr, n,
                                              ctypes.byref(nk))
        return st, nk.value

    def forward(self, weights: DeviceWeights, x, out, topk_ids=None, topk_w=None, workspace=None,
                stream=None, weights_struct: Optional[Weights] = None) -> None:
        """out[T, H] = layer(x[T, H]); tensors on the current device.  Raises on error."""
        import torch
        T = int(x.shape[0])
        if workspace is None:
            workspace = self.new_workspace(T, x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        ws = weights_struct if weights_struct is not None else weights.struct()
        st = self.forward_raw(ws, _ptr(x), T, _ptr(out), _ptr(topk_ids), _ptr(topk_w),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              stream.cuda_stream)
        if st != FLINT_OK:
            raise FlintError(st, f"flint_moe_forward: {status_string(st)}: {self.last_error()}")

    def forward_noalloc(self, weights: DeviceWeights, x, out, topk_ids=None, topk_w=None,
                        stream=None) -> None:
        """The layer with the library's static scratch array as workspace (T <= 64)."""
        import torch
        T = int(x.shape[0])
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        st = self.lib.flint_moe_forward_noalloc(self.handle, ctypes.byref(weights.struct()), _ptr(x),
                                                T, _ptr(out), _ptr(topk_ids), _ptr(topk_w),
                                                stream.cuda_stream)
        if st != FLINT_OK:
            raise FlintError(st, f"flint_moe_forward_noalloc: {status_string(st)}: "
                                 f"{self.last_error()}")

    def block_forward_raw(self, weights: Weights, gamma_ptr, eps, r_ptr, T, out_ptr, ids_ptr, w_ptr,
                          ws_ptr, ws_bytes, stream_ptr) -> int:
        """The pre-norm block's C call with raw addresses; returns the status code."""
        return self.lib.flint_moe_block_forward(self.handle, ctypes.byref(weights), gamma_ptr,
                                                float(eps), r_ptr, T, out_ptr, ids_ptr, w_ptr,
                                                ws_ptr, ws_bytes, stream_ptr)

    def block_forward_timed_raw(self, weights: Weights, gamma_ptr, eps, r_ptr, T, out_ptr, ids_ptr,
                                w_ptr, ws_ptr, ws_bytes, stream_ptr, event_handles) -> tuple:
        """The pre-norm block's timed C call; returns (status, number of kernels launched)."""
        n = len(event_handles)
        arr = (ctypes.c_void_p * n)(*event_handles)
        nk = ctypes.c_int32(0)
        st = self.lib.flint_moe_block_forward_timed(self.handle, ctypes.byref(weights), gamma_ptr,
                                                    float(eps), r_ptr, T, out_ptr, ids_ptr, w_ptr,
                                                    ws_ptr, ws_bytes, stream_ptr, arr, n,
                                                    ctypes.byref(nk))
        return st, nk.value

    def block_forward(self, weights: DeviceWeights, gamma, r, out, eps=1e-6, topk_ids=None,
                      topk_w=None, workspace=None, stream=None,
                      weights_struct: Optional[Weights] = None) -> None:
        """out[T, H] = r + layer(RMSNorm(r) * gamma), the pre-norm block.  Raises on error."""
        import torch
        T = int(r.shape[0])
        if workspace is None:
            workspace = self.new_workspace(T, r.device)
        if stream is None:
            stream = torch.cuda.current_stream(r.device)
        ws = weights_struct if weights_struct is not None else weights.struct()
        st = self.block_forward_raw(ws, _ptr(gamma), eps, _ptr(r), T, _ptr(out), _ptr(topk_ids),
                                    _ptr(topk_w), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), stream.cuda_stream)
        if st != FLINT_OK:
            raise FlintError(st, f"flint_moe_block_forward: {status_string(st)}: {self.last_error()}")

    def lowlat_forward_raw(self, weights: Weights, wo_ptr, attn_ptr, r_ptr, gamma_ptr,
                           gamma_next_ptr, eps, T, r_out_ptr, n_out_ptr, ids_ptr, w_ptr, ws_ptr,
                           ws_bytes, fused, stream_ptr) -> int:
        """The low-latency path's C call with raw addresses; returns the status code."""
        return self.lib.flint_moe_lowlat_forward(self.handle, ctypes.byref(weights), wo_ptr, attn_ptr,
                                                 r_ptr, gamma_ptr, gamma_next_ptr, float(eps), T,
                                                 r_out_ptr, n_out_ptr, ids_ptr, w_ptr, ws_ptr,
                                                 ws_bytes, int(fused), stream_ptr)

    def lowlat_forward_timed_raw(self, weights: Weights, wo_ptr, attn_ptr, r_ptr, gamma_ptr,
                                 gamma_next_ptr, eps, T, r_out_ptr, n_out_ptr, ids_ptr, w_ptr,
                                 ws_ptr, ws_bytes, fused, stream_ptr, event_handles) -> tuple:
        """The low-latency path's timed C call; returns (status, kernels launched)."""
        n = len(event_handles)
        arr = (ctypes.c_void_p * n)(*event_handles)
        nk = ctypes.c_int32(0)
        st = self.lib.flint_moe_lowlat_forward_timed(
            self.handle, ctypes.byref(weights), wo_ptr, attn_ptr, r_ptr, gamma_ptr, gamma_next_ptr,
            float(eps), T, r_out_ptr, n_out_ptr, ids_ptr, w_ptr, ws_ptr, ws_bytes, int(fused),
            stream_ptr, arr, n, ctypes.byref(nk))
        return st, nk.value

    def lowlat_forward(self, weights: DeviceWeights, wo, attn, r, gamma, r_out, gamma_next=None,
                       n_out=None, eps=1e-6, topk_ids=None, topk_w=None, workspace=None,
                       fused=True, stream=None) -> None:
        """r_out = r1 + layer(RMSNorm(r1) * gamma) with r1 = r + Wo attn, and
        n_out = RMSNorm(r_out) * gamma_next: the low-latency decode path.  Raises on error."""
        import torch
        T = int(r.shape[0])
        if workspace is None:
            workspace = self.new_workspace(T, r.device)
        if stream is None:
            stream = torch.cuda.current_stream(r.device)
        st = self.lowlat_forward_raw(weights.struct(), _ptr(wo), _ptr(attn), _ptr(r), _ptr(gamma),
                                     _ptr(gamma_next), eps, T, _ptr(r_out), _ptr(n_out),
                                     _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), fused,
                                     stream.cuda_stream)
        if st != FLINT_OK:
            raise FlintError(st, f"flint_moe_lowlat_forward: {status_string(st)}: {self.last_error()}")

    def new_workspace(self, T: int, device):
        """A zero-filled workspace for up to T tokens (the header must start at zero)."""
        import torch
        n = max(self.workspace_bytes(T), HEADER_BYTES)
        return torch.zeros(n, dtype=torch.uint8, device=device)


class FlintMLP:
    """The dense SwiGLU MLP of Flint's layers 0 and 1 (a ``flint_mlp_ctx``)."""

    def __init__(self, inter=14336, hidden=2048, max_tokens=64):
        self.lib = load_library()
        self.cfg = MlpConfig(hidden, inter, max_tokens)
        h = ctypes.c_void_p()
        st = self.lib.flint_mlp_init(ctypes.byref(self.cfg), ctypes.byref(h))
        if st != FLINT_OK:
            raise FlintError(st, f"flint_mlp_init: {status_string(st)}")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.flint_mlp_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, T: int) -> int:
        return int(self.lib.flint_mlp_workspace_bytes(self.handle, T))

    def workspace_layout(self, T: int) -> dict:
        L = MlpWsLayout()
        st = self.lib.flint_mlp_workspace_layout(self.handle, T, ctypes.byref(L))
        if st != FLINT_OK:
            raise FlintError(st, f"flint_mlp_workspace_layout: {status_string(st)}")
        return {n: getattr(L, n) for n, _ in MlpWsLayout._fields_}

    def last_error(self) -> str:
        return self.lib.flint_mlp_last_error(self.handle).decode()

    def new_workspace(self, T: int, device):
        import torch
        return torch.empty(max(self.workspace_bytes(T), 256), dtype=torch.uint8, device=device)

    def forward_raw(self, w13_ptr, w2_ptr, gamma_ptr, eps, x_ptr, T, out_ptr, ws_ptr, ws_bytes,
                    stream_ptr) -> int:
        return self.lib.flint_mlp_forward(self.handle, w13_ptr, w2_ptr, gamma_ptr, float(eps), x_ptr,
                                          T, out_ptr, ws_ptr, ws_bytes, stream_ptr)

    def forward_timed_raw(self, w13_ptr, w2_ptr, gamma_ptr, eps, x_ptr, T, out_ptr, ws_ptr,
                          ws_bytes, stream_ptr, event_handles) -> tuple:
        n = len(event_handles)
        arr = (ctypes.c_void_p * n)(*event_handles)
        nk = ctypes.c_int32(0)
        st = self.lib.flint_mlp_forward_timed(self.handle, w13_ptr, w2_ptr, gamma_ptr, float(eps),
                                              x_ptr, T, out_ptr, ws_ptr, ws_bytes, stream_ptr, arr,
                                              n, ctypes.byref(nk))
        return st, nk.value

    def forward(self, w13, w2, x, out, gamma=None, eps=1e-6, workspace=None, stream=None) -> None:
        """out = MLP(x), or x + MLP(RMSNorm(x) * gamma) when gamma is given.  Raises on error."""
        import torch
        T = int(x.shape[0])
        if workspace is None:
            workspace = self.new_workspace(T, x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        st = self.forward_raw(_ptr(w13), _ptr(w2), _ptr(gamma), eps, _ptr(x), T, _ptr(out),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              stream.cuda_stream)
        if st != FLINT_OK:
            raise FlintError(st, f"flint_mlp_forward: {status_string(st)}: {self.last_error()}")


def calib_stream_read(src_ptr: int, nbytes: int, sink_ptr: int, stream_ptr) -> None:
    """The streaming-read probe on raw addresses (see flint_moe_calib_stream_read)."""
    st = load_library().flint_moe_calib_stream_read(src_ptr, nbytes, sink_ptr, stream_ptr)
    if st != FLINT_OK:
        raise FlintError(st, f"flint_moe_calib_stream_read: {status_string(st)}")


def bf16_tensor(bits, device):
    """Upload a numpy uint16 array of bf16 bit patterns as a torch.bfloat16 tensor."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def bf16_bits(t):
    """Download a torch.bfloat16 tensor as numpy uint16 bit patterns."""
    import numpy as np
    return t.detach().contiguous().view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)

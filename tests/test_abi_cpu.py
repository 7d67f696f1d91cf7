"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host before anything is enqueued."""

import ctypes
import os
import re

import pytest

import sparse_expert_gemv_amd as sg
from sparse_expert_gemv_amd.flint_moe import Config, Weights, ExpertBank

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"\b(flint_(?:moe|mlp)_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = sg.load_library()
    decl = declared_symbols()
    assert decl, "no declarations found"
    assert decl == set(sg.ABI_SYMBOLS)
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings():
    assert sg.status_string(0) == "FLINT_OK"
    assert sg.status_string(3) == "FLINT_ERR_WORKSPACE"
    assert sg.status_string(99) == "FLINT_ERR_UNKNOWN"


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=1024), sg.FLINT_ERR_UNSUPPORTED),
    (dict(inter=256), sg.FLINT_ERR_UNSUPPORTED),
    (dict(n_experts=300), sg.FLINT_ERR_UNSUPPORTED),
    (dict(top_k=9, n_experts=16), sg.FLINT_ERR_UNSUPPORTED),
    (dict(top_k=7, n_experts=6), sg.FLINT_ERR_INVALID_ARG),
    (dict(max_tokens=0), sg.FLINT_ERR_INVALID_ARG),
    (dict(routed_scale=float("nan")), sg.FLINT_ERR_INVALID_ARG),
    (dict(fmt=7), sg.FLINT_ERR_INVALID_ARG),
    (dict(fmt=sg.FLINT_W_NVFP4, inter=1024), sg.FLINT_ERR_UNSUPPORTED),
])
def test_init_rejects(kw, status):
    with pytest.raises(sg.FlintError) as e:
        sg.FlintMoE(**kw)
    assert e.value.status == status


def test_init_null_and_destroy_null():
    lib = sg.load_library()
    assert lib.flint_moe_init(None, None) == sg.FLINT_ERR_INVALID_ARG
    lib.flint_moe_destroy(None)


def test_workspace_sizes_grow_with_T():
    m = sg.FlintMoE(max_tokens=64)
    assert m.workspace_bytes(0) == 0
    sizes = [m.workspace_bytes(T) for T in (1, 2, 8, 64)]
    assert sizes == sorted(sizes) and sizes[0] > sg.flint_moe.HEADER_BYTES
    lay = m.workspace_layout(8)
    offs = [lay[k] for k in ("header", "logits", "topk_ids", "topk_w", "route", "h", "extra")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay["route"] + (2 + 2 * 256 + 8 * 6) * 4 <= lay["h"]
    assert lay["logits"] - lay["header"] >= sg.flint_moe.HEADER_BYTES
    hdr_decl = re.search(r"FLINT_MOE_WS_HEADER_BYTES\s+(\d+)",
                         open(os.path.join(ROOT, "include", "flint_moe.h")).read())
    assert int(hdr_decl.group(1)) == sg.flint_moe.HEADER_BYTES
    assert lay["h"] + (8 * 6 + 8) * 512 * 4 <= lay["total_bytes"]


def _fake_weights(base=1 << 20):
    b = ExpertBank(base, base + 4096, None, None, None, None)
    return Weights(base + 8192, None, b, b)


def test_forward_host_validation_without_gpu():
    """Every one of these returns before any HIP call (no GPU needed)."""
    m = sg.FlintMoE(max_tokens=8)
    W = _fake_weights()
    x, out, ws = 1 << 30, 1 << 31, 1 << 32
    need = m.workspace_bytes(4)
    f = lambda **k: m.forward_raw(k.get("w", W), k.get("x", x), k.get("T", 4), k.get("out", out),
                                  None, None, k.get("ws", ws), k.get("nbytes", need), None)
    assert f(T=-1) == sg.FLINT_ERR_INVALID_ARG
    assert f(T=9) == sg.FLINT_ERR_INVALID_ARG and "max_tokens" in m.last_error()
    assert f(x=None) == sg.FLINT_ERR_INVALID_ARG
    assert f(x=x + 2) == sg.FLINT_ERR_INVALID_ARG and "aligned" in m.last_error()
    assert f(out=x + 4096) == sg.FLINT_ERR_INVALID_ARG and "overlaps" in m.last_error()
    assert f(ws=ws + 16) == sg.FLINT_ERR_INVALID_ARG
    assert f(nbytes=need - 1) == sg.FLINT_ERR_WORKSPACE
    bad = _fake_weights()
    bad.routed.w2 = None
    assert f(w=bad) == sg.FLINT_ERR_INVALID_ARG
    assert m.forward_raw(W, None, 0, None, None, None, None, 0, None) == sg.FLINT_OK
    m4 = sg.FlintMoE(max_tokens=8, fmt=sg.FLINT_W_NVFP4)
    need4 = m4.workspace_bytes(4)
    assert m4.forward_raw(W, x, 4, out, None, None, ws, need4, None) == sg.FLINT_ERR_INVALID_ARG
    assert "scales" in m4.last_error()
    b4 = ExpertBank(1 << 20, (1 << 20) + 4096, 1 << 24, (1 << 24) + 8, 1 << 25, (1 << 25) + 4)
    W4 = Weights((1 << 20) + 8192, None, b4, b4)
    assert m4.forward_raw(W4, x, 4, out, None, None, ws, need4, None) == sg.FLINT_ERR_INVALID_ARG
    assert "block scales must be 16-byte aligned" in m4.last_error()
    lib = sg.load_library()
    assert lib.flint_moe_forward(None, None, None, 1, None, None, None, None, 0, None) == \
        sg.FLINT_ERR_INVALID_ARG


def test_block_forward_host_validation_without_gpu():
    """The pre-norm block's own checks (gamma, eps, out vs r), all on the host."""
    m = sg.FlintMoE(max_tokens=8)
    W = _fake_weights()
    r, out, ws, g = 1 << 30, 1 << 31, 1 << 32, 1 << 29
    need = m.workspace_bytes(4)
    f = lambda **k: m.block_forward_raw(W, k.get("g", g), k.get("eps", 1e-6), k.get("r", r),
                                        k.get("T", 4), k.get("out", out), None, None, ws,
                                        k.get("nbytes", need), None)
    assert f(g=None) == sg.FLINT_ERR_INVALID_ARG and "gamma" in m.last_error()
    assert f(g=g + 8) == sg.FLINT_ERR_INVALID_ARG and "gamma" in m.last_error()
    assert f(eps=-1.0) == sg.FLINT_ERR_INVALID_ARG and "eps" in m.last_error()
    assert f(eps=float("nan")) == sg.FLINT_ERR_INVALID_ARG and "eps" in m.last_error()
    assert f(eps=float("inf")) == sg.FLINT_ERR_INVALID_ARG
    assert f(out=r + 2048) == sg.FLINT_ERR_INVALID_ARG and "overlaps r" in m.last_error()
    assert f(T=9) == sg.FLINT_ERR_INVALID_ARG
    assert f(nbytes=need - 1) == sg.FLINT_ERR_WORKSPACE
    assert f(T=0, g=None) == sg.FLINT_OK
    lib = sg.load_library()
    assert lib.flint_moe_block_forward(None, None, None, 0.0, None, 1, None, None, None, None, 0,
                                       None) == sg.FLINT_ERR_INVALID_ARG
    nk = ctypes.c_int32(0)
    assert m.block_forward_timed_raw(W, g, 1e-6, r, 4, out, None, None, ws, need, None,
                                     [None] * 4)[0] == sg.FLINT_ERR_INVALID_ARG


def test_noalloc_forward_host_validation_without_gpu():
    """The no-allocation forward rejects what its static scratch cannot hold
    before it touches the GPU."""
    m = sg.FlintMoE(max_tokens=128)
    W = _fake_weights()
    x, out = 1 << 30, 1 << 31
    lib = m.lib
    call = lambda T: lib.flint_moe_forward_noalloc(m.handle, ctypes.byref(W), x, T, out, None,
                                                   None, None)
    assert call(65) == sg.FLINT_ERR_UNSUPPORTED and "T <= 64" in m.last_error()
    assert call(129) == sg.FLINT_ERR_INVALID_ARG and "max_tokens" in m.last_error()
    assert call(-1) == sg.FLINT_ERR_INVALID_ARG
    assert call(0) == sg.FLINT_OK
    assert lib.flint_moe_forward_noalloc(None, None, None, 1, None, None, None, None) == \
        sg.FLINT_ERR_INVALID_ARG
    hdr = open(os.path.join(ROOT, "include", "flint_moe.h")).read()
    assert int(re.search(r"FLINT_MOE_NOALLOC_MAX_TOKENS\s+(\d+)", hdr).group(1)) == 64
    # The largest batch it takes fits its scratch array.
    scratch = int(re.search(r"FLINT_MOE_NOALLOC_SCRATCH_BYTES\s+(\d+)", hdr).group(1))
    assert sg.FlintMoE(max_tokens=64, top_k=8).workspace_bytes(64) <= scratch


def test_workspace_has_a_normed_region():
    m = sg.FlintMoE(max_tokens=8192)
    for T in (1, 8, 64, 65, 8192):
        lay = m.workspace_layout(T)
        assert lay["normed"] % 256 == 0
        assert lay["normed"] >= lay["route"] + (2 + 2 * 256 + T * 6) * 4
        assert lay["normed"] + T * 2048 * 2 <= min(v for k, v in lay.items()
                                                    if v > lay["normed"] or k == "total_bytes")


@pytest.mark.parametrize("kw,status", [
    (dict(inter=0), sg.FLINT_ERR_INVALID_ARG),
    (dict(inter=700), sg.FLINT_ERR_INVALID_ARG),
    (dict(inter=32768 + 512), sg.FLINT_ERR_INVALID_ARG),
    (dict(max_tokens=0), sg.FLINT_ERR_INVALID_ARG),
    (dict(hidden=1024), sg.FLINT_ERR_UNSUPPORTED),
])
def test_mlp_init_rejects(kw, status):
    with pytest.raises(sg.FlintError) as e:
        sg.FlintMLP(**kw)
    assert e.value.status == status


def test_mlp_workspace_and_host_validation_without_gpu():
    m = sg.FlintMLP(inter=1024, max_tokens=128)
    assert m.workspace_bytes(0) == 0
    lay = m.workspace_layout(8)
    assert lay["normed"] == 0 and lay["h"] >= 8 * 2048 * 2 and lay["h"] % 256 == 0
    assert lay["total_bytes"] >= lay["h"] + 8 * 1024 * 4          # fp32 h for T <= 64
    lay = m.workspace_layout(100)
    assert lay["total_bytes"] >= lay["h"] + 100 * 1024 * 2        # fp16 h above
    w13, w2, g, x, out, ws = 1 << 28, 1 << 29, 1 << 27, 1 << 30, 1 << 31, 1 << 32
    need = m.workspace_bytes(4)
    f = lambda **k: m.forward_raw(k.get("w13", w13), k.get("w2", w2), k.get("g", g),
                                  k.get("eps", 1e-6), k.get("x", x), k.get("T", 4),
                                  k.get("out", out), k.get("ws", ws), k.get("nbytes", need), None)
    assert f(T=-1) == sg.FLINT_ERR_INVALID_ARG
    assert f(T=129) == sg.FLINT_ERR_INVALID_ARG and "max_tokens" in m.last_error()
    assert f(w13=None) == sg.FLINT_ERR_INVALID_ARG
    assert f(w2=w2 + 8) == sg.FLINT_ERR_INVALID_ARG and "aligned" in m.last_error()
    assert f(g=g + 2) == sg.FLINT_ERR_INVALID_ARG and "gamma" in m.last_error()
    assert f(eps=-1.0) == sg.FLINT_ERR_INVALID_ARG and "eps" in m.last_error()
    assert f(out=x + 4096) == sg.FLINT_ERR_INVALID_ARG and "overlaps" in m.last_error()
    assert f(ws=ws + 64) == sg.FLINT_ERR_INVALID_ARG
    assert f(nbytes=need - 1) == sg.FLINT_ERR_WORKSPACE
    assert f(T=0, x=None) == sg.FLINT_OK
    assert m.forward_timed_raw(w13, w2, g, 1e-6, x, 4, out, ws, need, None, [None] * 3)[0] == \
        sg.FLINT_ERR_INVALID_ARG
    lib = sg.load_library()
    assert lib.flint_mlp_init(None, None) == sg.FLINT_ERR_INVALID_ARG
    lib.flint_mlp_destroy(None)

"""GPU parity of the NVFP4 (W4A16) decode path against the fp64 oracle.

Weights: the seeded bf16 layer encoded as E2M1 codes + E4M3 block scales
(one per 16 K-elements) + an fp32 tensor scale.  The oracle evaluates the
layer on the decoded weights (exact in fp64); the router, x and out stay
bf16.  Tolerance: max |err| <= 5e-2 * RMS(oracle output).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import OracleLayer, bf16_to_f64, moe_forward  # noqa: E402
from oracle.grading import TOL_NVFP4, grade  # noqa: E402
from synth import SyntheticLayer, make_x  # noqa: E402
from synth.device import nvfp4_layer, upload_nvfp4  # noqa: E402

pytestmark = pytest.mark.gpu
SEED = 0


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev4(flint_nvfp4):
    return flint_nvfp4


def run4(dev4, xb, bias=False):
    sg = dev4["sg"]
    T = xb.shape[0]
    moe = sg.FlintMoE(max_tokens=64, fmt=sg.FLINT_W_NVFP4)
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
    moe.forward(dev4["Wb"] if bias else dev4["W"], x, out, ids, w)
    torch.cuda.synchronize()
    return sg.bf16_bits(out), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,bias,x_seed", [(1, False, 0), (8, False, 0), (3, True, 1),
                                           (13, False, 2), (64, True, 3)])
def test_nvfp4_decode_matches_oracle(dev4, T, bias, x_seed):
    say(f"nvfp4 parity T={T} bias={bias} x_seed={x_seed}")
    xb = make_x(T, seed=SEED, x_seed=x_seed)
    out, ids, w = run4(dev4, xb, bias)
    res = moe_forward(dev4["Lb"] if bias else dev4["L"], xb)
    g = grade(out, ids, res, tol=TOL_NVFP4)
    print(g)
    assert g.ok, str(g)
    for t, r in enumerate(res):
        if t not in g.excluded:
            assert ids[t].tolist() == r.ids.tolist()
            np.testing.assert_allclose(w[t], r.weights, rtol=2e-6, atol=1e-7)
    if not bias:
        ref16 = moe_forward(dev4["L16"], xb)
        g16 = grade(out, ids, ref16, tol=1.0)
        print(f"against the bf16 layer (reported, not graded): ratio={g16.ratio:.3f}")


def test_nvfp4_rejects_missing_scales(dev4):
    sg = dev4["sg"]
    moe = sg.FlintMoE(max_tokens=8, fmt=sg.FLINT_W_NVFP4)
    W = dev4["W"].struct()
    W.routed.w13_scale = None
    x = torch.zeros((1, 2048), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    ws = moe.new_workspace(1, "cuda")
    st = moe.forward_raw(W, x.data_ptr(), 1, out.data_ptr(), None, None, ws.data_ptr(),
                         ws.numel(), None)
    assert st == sg.FLINT_ERR_INVALID_ARG


def test_nvfp4_intermediate_h(dev4):
    """h of every slot after the gate/up GEMV against the oracle's h.  With
    NVFP4 weights (W4A16) the kernels hand h to the down GEMV as bf16: each
    value is the oracle's to the fp32 accumulation error plus one bf16
    rounding (relative 2^-8 at most)."""
    sg = dev4["sg"]
    T = 2
    say("nvfp4 intermediates T=2")
    xb = make_x(T, seed=SEED, x_seed=5)
    moe = sg.FlintMoE(max_tokens=64, fmt=sg.FLINT_W_NVFP4)
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    moe.forward(dev4["W"], x, out, ids, None, ws)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(T)
    h = bf16_to_f64(ws[lay["h"]:lay["h"] + (T * 7) * 512 * 2].cpu().numpy().view(np.uint16)).reshape(T * 7, 512)
    res = moe_forward(dev4["L"], xb)
    for t, r in enumerate(res):
        sc = np.max(np.abs(r.h_shared))
        np.testing.assert_allclose(h[T * 6 + t], r.h_shared, rtol=2.0 ** -8, atol=1e-4 * sc,
                                   err_msg=f"shared h of token {t}")
        for j in range(6):
            sc = np.max(np.abs(r.h_routed[j]))
            np.testing.assert_allclose(h[t * 6 + j], r.h_routed[j], rtol=2.0 ** -8, atol=1e-4 * sc,
                                       err_msg=f"routed h of token {t} rank {j}")


@pytest.mark.parametrize("T,x_seed", [(1, 0), (8, 1)])
def test_nvfp4_block_matches_oracle(dev4, T, x_seed):
    """The pre-norm block over NVFP4 experts: out = r + layer(RMSNorm(r) * gamma)."""
    from oracle.block import block_forward
    from oracle.grading import grade_block
    from synth import make_residual
    sg = dev4["sg"]
    say(f"nvfp4 block parity T={T} x_seed={x_seed}")
    gamma = SyntheticLayer(SEED).norm_weight()
    rb = make_residual(T, seed=SEED, x_seed=x_seed)
    moe = sg.FlintMoE(max_tokens=64, fmt=sg.FLINT_W_NVFP4)
    r = sg.bf16_tensor(rb, "cuda")
    out = torch.empty_like(r)
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
    moe.block_forward(dev4["W"], sg.bf16_tensor(gamma, "cuda"), r, out, eps=1e-6,
                      topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    res = block_forward(dev4["L"], rb, gamma, eps=1e-6)
    g = grade_block(sg.bf16_bits(out), ids.cpu().numpy(), res, tol=TOL_NVFP4)
    print(g)
    assert g.ok, str(g)


@pytest.mark.parametrize("E,k", [(64, 8), (32, 1), (8, 8)])
def test_nvfp4_other_expert_counts(E, k):
    """Expert counts and top-k other than Flint's with NVFP4 weights, at the
    batch sizes of the small-batch down kernel (eight active experts per
    wave at T k > 48, six below) and past it; (8, 8) selects every expert."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_expert_gemv_amd as sg
    from synth import LayerShape
    say(f"nvfp4 layer E={E} k={k}")
    syn = SyntheticLayer(5, LayerShape(n_experts=E, top_k=k))
    syn.routed_banks()
    q = nvfp4_layer(syn)
    t = upload_nvfp4(syn, q, "cuda")

    def bank(name):
        return sg.DeviceBank(t[f"{name}_w13_q"], t[f"{name}_w2_q"], t[f"{name}_w13_s"],
                             t[f"{name}_w2_s"], t[f"{name}_w13_g"], t[f"{name}_w2_g"])

    W = sg.DeviceWeights(t["router_w"], None, bank("routed"), bank("shared"))

    def raw(e):
        b, i = ("shared", 0) if e < 0 else ("routed", e)
        d = q[b]
        return ((d["w13_q"][i], d["w13_s"][i], d["w13_g"][i]),
                (d["w2_q"][i], d["w2_s"][i], d["w2_g"][i]))

    L = OracleLayer(2048, E, k, 512, syn.router_w(), None, raw, fmt="nvfp4")
    moe = sg.FlintMoE(n_experts=E, top_k=k, max_tokens=16, fmt=sg.FLINT_W_NVFP4)
    for T in (2, 5, 7, 8, 13):
        say(f"  nvfp4 E={E} k={k} T={T}")
        xb = make_x(T, seed=5, x_seed=T)
        x = sg.bf16_tensor(xb, "cuda")
        out = torch.empty_like(x)
        ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
        moe.forward(W, x, out, ids, None, moe.new_workspace(T, "cuda"))
        torch.cuda.synchronize()
        g = grade(sg.bf16_bits(out), ids.cpu().numpy(), moe_forward(L, xb), tol=TOL_NVFP4)
        print(g)
        assert g.ok, f"E={E} k={k} T={T}: {g}"

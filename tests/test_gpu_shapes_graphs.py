"""GPU parity for other layer shapes, the router-weight flags on the prefill
path, and repeated HIP-graph replays.

* Expert counts and top-k other than Flint's (E 32/64/128, k 1/4/8; H and I
  stay 2048/512, the sizes the kernels are built for), decode and prefill.
* renormalize off and routed_scale != 1 on the prefill-sized path.
* A forward captured in a HIP graph and replayed several times, with new x
  between replays and eager forwards in between: every replay must equal the
  eager result bit for bit (the completion counters reset themselves).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import OracleLayer, moe_forward  # noqa: E402
from oracle.grading import TOL_BF16, grade  # noqa: E402
from synth import LayerShape, SyntheticLayer, make_x  # noqa: E402
from synth.device import upload_bf16  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def forward(sg, moe, W, xb, k):
    T = xb.shape[0]
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    moe.forward(W, x, out, ids, None, ws)
    torch.cuda.synchronize()
    return sg.bf16_bits(out), ids.cpu().numpy()


@pytest.mark.parametrize("E,k", [(64, 8), (32, 1), (128, 4), (8, 8), (1, 1)])
def test_other_expert_counts(E, k):
    """Other (E, k) than Flint's, through every routing path; (8, 8) selects
    every expert (k = E: the top-k keeps all of them, ranked), (1, 1) has a
    single routed expert that every token takes with weight 1."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_expert_gemv_amd as sg
    say(f"layer E={E} k={k}")
    syn = SyntheticLayer(3, LayerShape(n_experts=E, top_k=k))
    syn.routed_banks()
    t = upload_bf16(syn, "cuda")
    W = sg.DeviceWeights(t["router_w"], None, sg.DeviceBank(t["w13"], t["w2"]),
                         sg.DeviceBank(t["sh_w13"], t["sh_w2"]))
    L = OracleLayer(2048, E, k, 512, syn.router_w(), None, syn.expert)
    moe = sg.FlintMoE(n_experts=E, top_k=k, max_tokens=100)
    for T in (1, 4, 5, 13, 64, 100):   # routing in gate/up (T*k <= 16); 8-wave router; 16-wave router; prefill
        say(f"  E={E} k={k} T={T}")
        xb = make_x(T, seed=3, x_seed=T)
        out, ids = forward(sg, moe, W, xb, k)
        g = grade(out, ids, moe_forward(L, xb), tol=TOL_BF16)
        print(g)
        assert g.ok, f"E={E} k={k} T={T}: {g}"


def test_prefill_flags(flint_bf16):
    sg = flint_bf16["sg"]
    say("prefill T=100 renormalize off, routed_scale 2.5")
    moe = sg.FlintMoE(max_tokens=100, renormalize=False, routed_scale=2.5)
    xb = make_x(100, seed=0, x_seed=11)
    out, ids = forward(sg, moe, flint_bf16["Wb"], xb, 6)
    g = grade(out, ids, moe_forward(flint_bf16["Lb"], xb, renormalize=False, routed_scale=2.5),
              tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)


@pytest.mark.parametrize("T", [1, 8, 32, 300])   # routing in gate/up; 4-wave; 16-wave router; prefill
def test_graph_replays_match_eager(flint_bf16, T):
    sg = flint_bf16["sg"]
    say(f"graph replays T={T}")
    moe = sg.FlintMoE(max_tokens=T)
    W = flint_bf16["W"]
    x = sg.bf16_tensor(make_x(T, seed=0, x_seed=0), "cuda")
    out = torch.empty_like(x)
    ids = torch.empty((T, 6), dtype=torch.int32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    # Eager reference outputs and ids for four different inputs.
    xs = [sg.bf16_tensor(make_x(T, seed=0, x_seed=20 + r), "cuda") for r in range(4)]
    ref = []
    for xr in xs:
        x.copy_(xr)
        moe.forward(W, x, out, ids, None, ws)
        torch.cuda.synchronize()
        ref.append((out.clone(), ids.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.forward(W, x, out, ids, None, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = moe.forward_raw(W.struct(), int(x.data_ptr()), T, int(out.data_ptr()),
                             int(ids.data_ptr()), 0, int(ws.data_ptr()), ws.numel(),
                             torch.cuda.current_stream().cuda_stream)
        assert st == sg.FLINT_OK
    for rep in range(2):
        for r, xr in enumerate(xs):
            x.copy_(xr)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref[r][0]), f"replay {rep}/{r}: output differs from eager"
            assert torch.equal(ids, ref[r][1]), f"replay {rep}/{r}: ids differ from eager"
            # eager work between replays
            moe.forward(W, x, out, ids, None, ws)
            torch.cuda.synchronize()
            assert torch.equal(out, ref[r][0])


def _replay_check(call_eager, call_raw, set_input, outs, n_inputs=3):
    """Eager results for n inputs, then a captured graph of one call replayed
    twice per input with eager work in between: every replay bit-equal."""
    ref = []
    for r in range(n_inputs):
        set_input(r)
        call_eager()
        torch.cuda.synchronize()
        ref.append([o.clone() for o in outs])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call_eager()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert call_raw(torch.cuda.current_stream().cuda_stream) == 0
    for rep in range(2):
        for r in range(n_inputs):
            set_input(r)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for o, e in zip(outs, ref[r]):
                assert torch.equal(o, e), f"replay {rep}/{r} differs from eager"
            call_eager()
            torch.cuda.synchronize()


@pytest.mark.parametrize("T", [8, 100])
def test_block_graph_replays_match_eager(flint_bf16, T):
    """The pre-norm block (norm fused into the router launch for T <= 64, its
    own launch above) under graph capture."""
    from synth import make_residual
    sg = flint_bf16["sg"]
    say(f"pre-norm block graph replays T={T}")
    moe = sg.FlintMoE(max_tokens=T)
    W = flint_bf16["W"]
    gamma = sg.bf16_tensor(flint_bf16["syn"].norm_weight(), "cuda")
    r = sg.bf16_tensor(make_residual(T, seed=0, x_seed=0), "cuda")
    rs = [sg.bf16_tensor(make_residual(T, seed=0, x_seed=30 + i), "cuda") for i in range(3)]
    out = torch.empty_like(r)
    ids = torch.empty((T, 6), dtype=torch.int32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    Ws = W.struct()
    _replay_check(
        lambda: moe.block_forward(W, gamma, r, out, eps=1e-6, topk_ids=ids, workspace=ws),
        lambda s: moe.block_forward_raw(Ws, int(gamma.data_ptr()), 1e-6, int(r.data_ptr()), T,
                                        int(out.data_ptr()), int(ids.data_ptr()), 0,
                                        int(ws.data_ptr()), ws.numel(), s),
        lambda i: r.copy_(rs[i]), [out, ids])


@pytest.mark.parametrize("T,block", [(8, False), (8, True), (100, True)])
def test_dense_mlp_graph_replays_match_eager(T, block):
    from synth import SyntheticDenseMLP
    import sparse_expert_gemv_amd as sg
    say(f"dense MLP graph replays T={T} block={block}")
    S = SyntheticDenseMLP(seed=1, inter=1024)
    w13, w2 = sg.bf16_tensor(S.w13(), "cuda"), sg.bf16_tensor(S.w2(), "cuda")
    gamma = sg.bf16_tensor(S.norm_weight(), "cuda") if block else None
    m = sg.FlintMLP(inter=1024, max_tokens=T)
    x = sg.bf16_tensor(make_x(T, seed=0, x_seed=0), "cuda")
    xs = [sg.bf16_tensor(make_x(T, seed=0, x_seed=40 + i), "cuda") for i in range(3)]
    out = torch.empty_like(x)
    ws = m.new_workspace(T, "cuda")
    gp = int(gamma.data_ptr()) if block else None
    _replay_check(
        lambda: m.forward(w13, w2, x, out, gamma=gamma, workspace=ws),
        lambda s: m.forward_raw(int(w13.data_ptr()), int(w2.data_ptr()), gp, 1e-6, int(x.data_ptr()),
                                T, int(out.data_ptr()), int(ws.data_ptr()), ws.numel(), s),
        lambda i: x.copy_(xs[i]), [out])

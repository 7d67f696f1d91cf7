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


@pytest.mark.parametrize("E,k", [(64, 8), (32, 1), (128, 4)])
def test_other_expert_counts(E, k):
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
    for T in (1, 13, 64, 100):
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


@pytest.mark.parametrize("T", [8, 300])
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

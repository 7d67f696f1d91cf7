"""GPU parity of the prefill-sized (T > 64) MFMA path against the fp64 oracle.

Small T: every token against the per-token oracle.  T = 8192 (the prefill
workload, "RecursiveSI/flint — vLLM serving recipe", section "Benchmarking",
prefill 8K): the router output (ids, weights), the routing table and the
layer output of every token, against the expert-grouped oracle
(``oracle.grouped``, pinned token by token against the per-token oracle).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bucket, moe_forward  # noqa: E402
from oracle.grading import TOL_BF16, grade, grade_arrays  # noqa: E402
from oracle.grouped import moe_forward_grouped  # noqa: E402
from synth import make_x  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run(dev, xb, bias=False, max_tokens=8192):
    sg = dev["sg"]
    T = xb.shape[0]
    moe = sg.FlintMoE(max_tokens=max_tokens)
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    moe.forward(dev["Wb"] if bias else dev["W"], x, out, ids, w, ws)
    torch.cuda.synchronize()
    return dict(out=sg.bf16_bits(out), ids=ids.cpu().numpy(), w=w.cpu().numpy(), ws=ws, moe=moe)


@pytest.mark.parametrize("T,bias,x_seed", [(65, False, 0), (130, True, 1), (300, False, 2)])
def test_prefill_matches_oracle(flint_bf16, T, bias, x_seed):
    say(f"prefill parity T={T} bias={bias}")
    xb = make_x(T, seed=0, x_seed=x_seed)
    r = run(flint_bf16, xb, bias)
    res = moe_forward(flint_bf16["Lb"] if bias else flint_bf16["L"], xb)
    g = grade(r["out"], r["ids"], res, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)
    for t, rr in enumerate(res):
        if t not in g.excluded:
            assert r["ids"][t].tolist() == rr.ids.tolist()
            np.testing.assert_allclose(r["w"][t], rr.weights, rtol=2e-6, atol=1e-7)


def test_prefill_t8192_full(flint_bf16):
    T = 8192
    say("prefill T=8192: routing, table and output of every token")
    xb = make_x(T, seed=0, x_seed=0)
    r = run(flint_bf16, xb)
    G = moe_forward_grouped(flint_bf16["L"], xb)
    keep = G.gaps >= 1e-5
    print(f"excluded tokens (gap < 1e-5): {int((~keep).sum())}")
    assert np.array_equal(r["ids"][keep], G.ids[keep])
    np.testing.assert_allclose(r["w"][keep], G.weights[keep], rtol=2e-6, atol=1e-7)
    # Routing table: the bucketing of the device's own ids, bit-exact.
    b = bucket(r["ids"], 256)
    lay = r["moe"].workspace_layout(T)
    n_ints = 2 + 2 * 256 + T * 6
    route = r["ws"][lay["route"]:lay["route"] + 4 * n_ints].cpu().numpy().view(np.int32)
    nU = len(b["active"])
    assert route[0] == nU
    np.testing.assert_array_equal(route[1:1 + nU], b["active"])
    np.testing.assert_array_equal(route[1 + 256:1 + 256 + nU + 1],
                                  b["offsets"][b["active"].tolist() + [256]])
    np.testing.assert_array_equal(route[2 + 512:], b["slots"])
    # The output of every token.
    g = grade_arrays(r["out"], r["ids"], G.out, G.ids, G.gaps, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)
    assert g.n_graded == int(keep.sum())
    # The whole workspace header is zero again after the forward, and a
    # second forward gives the same bits.
    from sparse_expert_gemv_amd.flint_moe import HEADER_BYTES
    hdr = r["ws"][lay["header"]:lay["header"] + HEADER_BYTES].cpu().numpy().view(np.uint32)
    assert not hdr.any(), np.nonzero(hdr)
    r2 = run(flint_bf16, xb)
    np.testing.assert_array_equal(r2["out"], r["out"])


def test_prefill_ragged_beyond_the_workload(flint_bf16):
    """T = 12289 = 3 * 4096 + 1: half again the prefill workload and a multiple
    of no tile (32-token router blocks, 256-slot M-tiles, the bucketing's
    token parts), so every launch ends on a ragged tile.  Every token against
    the expert-grouped oracle."""
    T = 12289
    say("prefill T=12289: ragged tiles beyond the 8K workload")
    xb = make_x(T, seed=0, x_seed=7)
    r = run(flint_bf16, xb, max_tokens=T)
    G = moe_forward_grouped(flint_bf16["L"], xb)
    keep = G.gaps >= 1e-5
    assert np.array_equal(r["ids"][keep], G.ids[keep])
    np.testing.assert_allclose(r["w"][keep], G.weights[keep], rtol=2e-6, atol=1e-7)
    g = grade_arrays(r["out"], r["ids"], G.out, G.ids, G.gaps, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)
    assert g.n_graded == int(keep.sum())


def test_prefill_multi_tile_groups(flint_bf16):
    """Skewed routing (the router bias): slot groups that span several
    256-slot M-tiles (the largest has over 1300 slots).  Every token against
    the expert-grouped oracle."""
    T = 2048
    say("prefill T=2048 with router bias: multi-tile expert groups")
    xb = make_x(T, seed=0, x_seed=1)
    r = run(flint_bf16, xb, bias=True)
    counts = np.bincount(r["ids"].ravel(), minlength=256)
    assert counts.max() > 3 * 256, counts.max()
    G = moe_forward_grouped(flint_bf16["Lb"], xb)
    g = grade_arrays(r["out"], r["ids"], G.out, G.ids, G.gaps, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)


def test_prefill_deterministic(flint_bf16):
    say("prefill determinism T=1000")
    xb = make_x(1000, seed=0, x_seed=3)
    a = run(flint_bf16, xb)
    b = run(flint_bf16, xb)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["ids"], b["ids"])


def test_decode_and_prefill_agree_at_the_boundary(flint_bf16):
    """T = 64 (decode kernels) and T = 65 (prefill kernels) on the same first 64
    tokens: same routing, both within tolerance of the oracle."""
    say("decode/prefill boundary")
    xb = make_x(65, seed=0, x_seed=4)
    d = run(flint_bf16, xb[:64], max_tokens=64)
    p = run(flint_bf16, xb)
    np.testing.assert_array_equal(d["ids"], p["ids"][:64])
    res = moe_forward(flint_bf16["L"], xb[:64])
    for out in (d["out"], p["out"][:64]):
        g = grade(out, d["ids"], res)
        assert g.ok, str(g)


def _scaled_bits(bits, factor):
    from oracle import bf16_to_f64
    from oracle.block import f64_to_bf16_bits
    return f64_to_bf16_bits(bf16_to_f64(bits) * factor).reshape(bits.shape)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_prefill_large_activations_past_fp16_range(flint_bf16):
    """Every gate/up weight times 2^8 (exact in bf16): |h| reaches ~1e6 and
    |y| ~1e5, far past fp16's 65504; the prefill path's biased fp16
    intermediates keep them.  A 16-expert layer, T = 300, every token."""
    import sparse_expert_gemv_amd as sg
    from oracle import OracleLayer
    from synth import LayerShape, SyntheticLayer
    say("prefill with |h| past the fp16 range, T=300, 16 experts")
    S = SyntheticLayer(3, LayerShape(n_experts=16))
    w13 = np.stack([_scaled_bits(S.w13(e), 256.0) for e in range(16)])
    w2 = np.stack([S.w2(e) for e in range(16)])
    sh13, sh2 = _scaled_bits(S.w13(-1), 256.0), S.w2(-1)
    t = lambda b: sg.bf16_tensor(b, "cuda")
    W = sg.DeviceWeights(t(S.router_w()), None, sg.DeviceBank(t(w13), t(w2)),
                         sg.DeviceBank(t(sh13[None]), t(sh2[None])))
    L = OracleLayer(2048, 16, 6, 512, S.router_w(), None,
                    lambda e: (w13[e], w2[e]) if e >= 0 else (sh13, sh2))
    T = 300
    xb = make_x(T, seed=3, x_seed=1)
    moe = sg.FlintMoE(n_experts=16, max_tokens=T)
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    moe.forward(W, x, out, ids, None, moe.new_workspace(T, "cuda"))
    torch.cuda.synchronize()
    res = moe_forward(L, xb)
    h_max = max(max(np.max(np.abs(r.h_routed)), np.max(np.abs(r.h_shared))) for r in res)
    print(f"max |h| = {h_max:.3e}")
    assert h_max > 4 * 65504
    g = grade(sg.bf16_bits(out), ids.cpu().numpy(), res, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)

"""GPU parity of the prefill-sized (T > 64) MFMA path against the fp64 oracle.

Small T: every token against the oracle.  T = 8192 (the prefill workload):
the router output (ids, weights) and the routing table for every token, and
the layer output on a spread sample of tokens computed one by one by the
oracle.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bucket, moe_forward, route_all  # noqa: E402
from oracle.grading import TOL_BF16, grade  # noqa: E402
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


def test_prefill_t8192_sampled(flint_bf16):
    T = 8192
    say("prefill T=8192: routing of every token, output of a sample")
    xb = make_x(T, seed=0, x_seed=0)
    r = run(flint_bf16, xb)
    ids_ref, w_ref, gaps, _ = route_all(flint_bf16["L"], xb)
    keep = gaps >= 1e-5
    print(f"excluded tokens (gap < 1e-5): {int((~keep).sum())}")
    assert np.array_equal(r["ids"][keep], ids_ref[keep])
    np.testing.assert_allclose(r["w"][keep], w_ref[keep], rtol=2e-6, atol=1e-7)
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
    # Output of 48 tokens spread over the batch (first, last, tile edges).
    sample = sorted(set([0, 1, 63, 64, 65, 127, 4095, 4096, 8127, 8128, 8190, 8191] +
                        [int(v) for v in np.random.default_rng(0).choice(T, 36, replace=False)]))
    res = moe_forward(flint_bf16["L"], xb, tokens=sample)
    g = grade(r["out"], r["ids"], res, tokens=sample, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)


def test_prefill_multi_tile_groups(flint_bf16):
    """Skewed routing (the router bias): slot groups that span several
    256-slot M-tiles (the largest has over 1300 slots).  Tokens on both sides
    of every tile edge of the four largest groups, their last tokens and a
    random sample against the oracle."""
    T = 2048
    say("prefill T=2048 with router bias: multi-tile expert groups")
    xb = make_x(T, seed=0, x_seed=1)
    r = run(flint_bf16, xb, bias=True)
    counts = np.bincount(r["ids"].ravel(), minlength=256)
    big = np.argsort(counts)[::-1][:4]
    assert counts[big[0]] > 3 * 256, counts[big[0]]
    sample = set(np.random.default_rng(1).choice(T, 24, replace=False).tolist())
    for e in big:
        toks = np.nonzero((r["ids"] == e).any(axis=1))[0]   # the group's slot order
        for edge in range(256, len(toks), 256):
            sample.update((int(toks[edge - 1]), int(toks[edge])))
        sample.add(int(toks[-1]))
    sample = sorted(sample)
    res = moe_forward(flint_bf16["Lb"], xb, tokens=sample)
    g = grade(r["out"], r["ids"], res, tokens=sample, tol=TOL_BF16)
    print(f"{len(sample)} tokens: {g}")
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

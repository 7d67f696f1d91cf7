"""GPU parity of the pre-norm block (RMSNorm + layer + residual add) against
the fp64 oracle, through the C ABI, on both paths (decode T <= 64 with the
norm fused into the router launch; prefill with its own norm launch).

What is compared:
  * n, the normalised bf16 input the layer ran on (workspace region
    ``normed``): bit-exact, except that an element whose exact value lies
    within 1e-5 (relative) of a bf16 rounding midpoint may land on either
    neighbour (the kernel decides the rounding in fp32, the oracle in fp64);
  * the selected experts and their routing weights;
  * out = r + layer(n): |out - oracle| <= 2e-2 * RMS(oracle layer part)
    + 2^-8 |oracle out| (the second term is the bf16 rounding of the sum).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bf16_to_f64  # noqa: E402
from oracle.block import block_forward  # noqa: E402
from oracle.grading import TOL_BF16, grade_block, grade_block_arrays  # noqa: E402
from oracle.grouped import block_forward_grouped  # noqa: E402
from synth import make_residual  # noqa: E402

pytestmark = pytest.mark.gpu

EPS = 1e-6


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_block(dev, rb, gamma_bits, bias=False, max_tokens=64, eps=EPS):
    sg = dev["sg"]
    T = rb.shape[0]
    moe = sg.FlintMoE(max_tokens=max_tokens)
    r = sg.bf16_tensor(rb, "cuda")
    g = sg.bf16_tensor(gamma_bits, "cuda")
    out = torch.empty_like(r)
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    moe.block_forward(dev["Wb"] if bias else dev["W"], g, r, out, eps=eps, topk_ids=ids,
                      topk_w=w, workspace=ws)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(T)
    normed = ws[lay["normed"]:lay["normed"] + T * 2048 * 2].cpu().numpy().view(np.uint16)
    return dict(out=sg.bf16_bits(out), ids=ids.cpu().numpy(), w=w.cpu().numpy(),
                normed=normed.reshape(T, 2048), ws=ws, moe=moe, lay=lay)


def check_normed(got, ref_bits, ref_f64):
    """got / ref_bits: bf16 bits [H]; ref_f64: the oracle's unrounded n [H]."""
    d = got != ref_bits
    if not d.any():
        return 0
    gi, ri = got[d].astype(np.int32), ref_bits[d].astype(np.int32)
    assert np.all(np.abs(gi - ri) == 1), "normalised input differs by more than one bf16 step"
    a, b = bf16_to_f64(got[d]), bf16_to_f64(ref_bits[d])
    mid = (a + b) / 2
    v = ref_f64[d]
    assert np.all(np.abs(v - mid) <= 1e-5 * np.abs(v)), "a differing element is not at a midpoint"
    return int(d.sum())


def check_all(r, res, tol=TOL_BF16):
    g = grade_block(r["out"], r["ids"], res, tol=tol)
    print(g)
    assert g.ok, str(g)
    flips = [check_normed(r["normed"][t], rr.normed_bits, rr.normed_f64) for t, rr in enumerate(res)]
    assert sum(flips) <= max(4, len(res) * 2048 // 1000), f"{sum(flips)} midpoint flips"
    for t, rr in enumerate(res):
        if t in g.excluded:
            continue
        assert r["ids"][t].tolist() == rr.ids.tolist()
        # A token whose n took a different midpoint rounding routes on slightly
        # different logits (one bf16 step of one element moves a logit by up
        # to |Wr| * 2^-8 |n|): its weights get a looser bound.
        rtol = 2e-6 if flips[t] == 0 else 1e-4
        np.testing.assert_allclose(r["w"][t], rr.moe.weights, rtol=rtol, atol=1e-7)
    return g


@pytest.mark.parametrize("T,bias,x_seed", [(1, False, 0), (8, False, 0), (13, True, 1),
                                           (32, True, 2), (64, False, 3)])
def test_block_decode_matches_oracle(flint_bf16, T, bias, x_seed):
    say(f"block decode parity T={T} bias={bias} x_seed={x_seed}")
    dev = flint_bf16
    gamma = dev["syn"].norm_weight()
    rb = make_residual(T, seed=0, x_seed=x_seed)
    r = run_block(dev, rb, gamma, bias)
    res = block_forward(dev["Lb"] if bias else dev["L"], rb, gamma, eps=EPS)
    check_all(r, res)


@pytest.mark.parametrize("T,x_seed", [(65, 0), (300, 1)])
def test_block_prefill_matches_oracle(flint_bf16, T, x_seed):
    say(f"block prefill parity T={T} x_seed={x_seed}")
    dev = flint_bf16
    gamma = dev["syn"].norm_weight()
    rb = make_residual(T, seed=0, x_seed=x_seed)
    r = run_block(dev, rb, gamma, max_tokens=8192)
    res = block_forward(dev["L"], rb, gamma, eps=EPS)
    check_all(r, res)


def test_block_prefill_t8192_full(flint_bf16):
    """The prefill workload's size: n, ids, weights and out of every token,
    against the expert-grouped oracle."""
    T = 8192
    say("block prefill T=8192: every token")
    dev = flint_bf16
    gamma = dev["syn"].norm_weight()
    rb = make_residual(T, seed=0, x_seed=7)
    r = run_block(dev, rb, gamma, max_tokens=T)
    G = block_forward_grouped(dev["L"], rb, gamma, eps=EPS)
    flips = [check_normed(r["normed"][t], G.normed_bits[t], G.normed_f64[t]) for t in range(T)]
    assert sum(flips) <= T * 2048 // 1000, f"{sum(flips)} midpoint flips"
    g = grade_block_arrays(r["out"], r["ids"], G.out, G.layer_out, G.ids, G.gaps, tol=TOL_BF16)
    print(g)
    assert g.ok, str(g)
    keep = (G.gaps >= 1e-5) & (np.array(flips) == 0)
    assert np.array_equal(r["ids"][keep], G.ids[keep])
    np.testing.assert_allclose(r["w"][keep], G.weights[keep], rtol=2e-6, atol=1e-7)


def test_block_zero_gamma_returns_r_exactly(flint_bf16):
    """gamma = 0: n = 0, every expert's h is silu(0) * 0 = 0, so out = r bit for
    bit; all scores tie at sigmoid(0), so the lowest six indices are chosen."""
    say("block with zero gamma, T=5 and T=70")
    dev = flint_bf16
    for T, mt in ((5, 64), (70, 8192)):
        rb = make_residual(T, seed=0, x_seed=11)
        r = run_block(dev, rb, np.zeros(2048, np.uint16), max_tokens=mt)
        assert np.array_equal(r["out"], rb)
        assert not np.any(r["normed"] & np.uint16(0x7FFF))
        assert (r["ids"] == np.arange(6)).all()
        np.testing.assert_allclose(r["w"], 1.0 / 6, rtol=1e-6)


def test_block_equals_layer_on_its_own_normalised_input(flint_bf16):
    """Fusion check, GPU against GPU: the bare layer run on the block's n
    selects the same experts with the same weights and produces the same h,
    bit for bit (the router launch's in-register norm feeds the same bf16
    values that the gate/up launch reads back)."""
    say("block vs bare layer on the block's own n, T=8 and T=64")
    dev = flint_bf16
    sg = dev["sg"]
    gamma = dev["syn"].norm_weight()
    for T in (8, 64):
        rb = make_residual(T, seed=0, x_seed=5)
        r = run_block(dev, rb, gamma)
        moe = sg.FlintMoE(max_tokens=64)
        x = sg.bf16_tensor(r["normed"], "cuda")
        out = torch.empty_like(x)
        ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
        w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
        ws = moe.new_workspace(T, "cuda")
        moe.forward(dev["W"], x, out, ids, w, ws)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), r["ids"])
        assert np.array_equal(w.cpu().numpy(), r["w"])
        lay = moe.workspace_layout(T)
        nh = (T * 7) * 512 * 4
        h_bare = ws[lay["h"]:lay["h"] + nh].cpu().numpy()
        h_blk = r["ws"][r["lay"]["h"]:r["lay"]["h"] + nh].cpu().numpy()
        assert np.array_equal(h_bare, h_blk)

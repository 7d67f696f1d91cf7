"""GPU parity of the low-latency decode path (flint_moe_lowlat_forward: the
attention output projection with its residual add, the pre-norm MoE block and
the next layer's norm, fused into three launches, or the same arithmetic in
five) against the fp64 oracle (``oracle.decoder``), through the C ABI.

What is compared, per token:
  * r1 = bf16(r + Wo a), left in the workspace: equal to the oracle's bits,
    except where the exact value lies within the fp32 accumulation error
    (2^-17 sum_k |Wo a| + 2^-23 |r1|) of another rounding: near a midpoint,
    or, after cancellation, at tiny values;
  * n, ids, weights and r_out against the oracle run on the device's own r1
    (so that such a flip does not move the rest): n bit-exact up to midpoint
    flips, ids in rank order, weights to 2e-6, r_out within 2e-2 x RMS(layer
    part) + 2^-8 |r_out|;
  * n_out against the RMSNorm of the device's own r_out: bit-exact up to
    midpoint flips;
  * the fused and the five-launch forms bit for bit, and every completed
    forward leaves the workspace counters at zero with no expired wait.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bf16_to_f64  # noqa: E402
from oracle.block import block_token, f64_to_bf16_bits, rmsnorm  # noqa: E402
from oracle.decoder import decoder_forward  # noqa: E402
from oracle.grading import TOL_BF16, TOL_NVFP4, grade_block  # noqa: E402
from synth import make_attn, make_next_gain, make_o_proj, make_residual  # noqa: E402

pytestmark = pytest.mark.gpu
EPS = 1e-6
HDR_WORDS = 21504 // 4


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def attn_side(flint_bf16):
    sg = flint_bf16["sg"]
    wo = make_o_proj(seed=0)
    return dict(wo=wo, wo_dev=sg.bf16_tensor(wo, "cuda"), gnext=make_next_gain(seed=0))


def run(dev, side, T, x_seed, fused, with_next=True, bias=False):
    sg = dev["sg"]
    moe = sg.FlintMoE(max_tokens=8, fmt=dev.get("fmt", sg.FLINT_W_BF16))
    attn = make_attn(T, seed=0, x_seed=x_seed)
    rb = make_residual(T, seed=0, x_seed=x_seed)
    gamma = dev["syn"].norm_weight()
    d = lambda b: sg.bf16_tensor(b, "cuda")
    r_out = torch.empty((T, 2048), dtype=torch.bfloat16, device="cuda")
    n_out = torch.empty_like(r_out) if with_next else None
    ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
    ws = moe.new_workspace(T, "cuda")
    moe.lowlat_forward(dev["Wb"] if bias else dev["W"], side["wo_dev"], d(attn), d(rb), d(gamma),
                       r_out, gamma_next=d(side["gnext"]) if with_next else None, n_out=n_out,
                       eps=EPS, topk_ids=ids, topk_w=w, workspace=ws, fused=fused)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(T)
    region = lambda off, n: ws[off:off + n].cpu().numpy()
    return dict(attn=attn, rb=rb, gamma=gamma, r_out=sg.bf16_bits(r_out),
                n_out=None if n_out is None else sg.bf16_bits(n_out), ids=ids.cpu().numpy(),
                w=w.cpu().numpy(),
                r1=region(lay["resid1"], T * 4096).view(np.uint16).reshape(T, 2048),
                n=region(lay["normed"], T * 4096).view(np.uint16).reshape(T, 2048),
                header=region(0, HDR_WORDS * 4).view(np.uint32))


def flips_at_midpoints(got, ref_bits, ref_f64, slack):
    """Number of elements where got != ref.  Each must be a rounding of some
    value within `slack` (absolute, per element) of the exact one: bf16
    rounding is monotone, so got must lie between the roundings of
    exact - slack and exact + slack."""
    d = got != ref_bits
    if not d.any():
        return 0
    v, sl = ref_f64[d], np.broadcast_to(slack, got.shape)[d]
    lo = bf16_to_f64(f64_to_bf16_bits(v - sl))
    hi = bf16_to_f64(f64_to_bf16_bits(v + sl))
    g = bf16_to_f64(got[d])
    assert np.all((lo <= g) & (g <= hi)), "a differing element is beyond the rounding of its error bound"
    return int(d.sum())


def check(dev, side, r, bias=False):
    L = dev["Lb"] if bias else dev["L"]
    tol = TOL_NVFP4 if dev.get("fmt", 0) == dev["sg"].FLINT_W_NVFP4 else TOL_BF16
    T = r["rb"].shape[0]
    gnext = side["gnext"] if r["n_out"] is not None else None
    res = decoder_forward(L, side["wo"], r["attn"], r["rb"], r["gamma"], gnext, eps=EPS)
    # r1: fp32 accumulation of 4096 products against the fp64 sum.
    wo = bf16_to_f64(side["wo"]).reshape(2048, 4096)
    total_flips = 0
    for t in range(T):
        mag = np.abs(wo) @ np.abs(bf16_to_f64(r["attn"][t]))
        slack = 2.0 ** -17 * mag + 2.0 ** -23 * np.abs(res[t].r1_f64)
        total_flips += flips_at_midpoints(r["r1"][t], res[t].r1_bits, res[t].r1_f64, slack)
    assert total_flips <= max(4, T * 2048 // 200), f"{total_flips} r1 midpoint flips"
    # The block on the device's own r1.
    blk = [block_token(L, r["r1"][t], r["gamma"], EPS) for t in range(T)]
    g = grade_block(r["r_out"], r["ids"], blk, tol=tol)
    print(g)
    assert g.ok, str(g)
    for t, b in enumerate(blk):
        nflip = flips_at_midpoints(r["n"][t], b.normed_bits, b.normed_f64, 1e-5 * np.abs(b.normed_f64))
        assert nflip <= 4
        if t in g.excluded:
            continue
        assert r["ids"][t].tolist() == b.ids.tolist()
        # A token whose n took the other rounding at a midpoint routes on
        # slightly different logits: its weights get a looser bound.
        np.testing.assert_allclose(r["w"][t], b.moe.weights, rtol=2e-6 if nflip == 0 else 1e-4,
                                   atol=1e-7)
    # End to end against the oracle from the inputs (r1 flips included).
    g2 = grade_block(r["r_out"], r["ids"], [x.block for x in res], tol=tol)
    print("end to end:", g2)
    assert g2.ok, str(g2)
    if r["n_out"] is not None:
        for t in range(T):
            n64 = rmsnorm(bf16_to_f64(r["r_out"][t]), bf16_to_f64(gnext), EPS)
            assert flips_at_midpoints(r["n_out"][t], f64_to_bf16_bits(n64), n64,
                                      1e-5 * np.abs(n64)) <= 4
    assert not r["header"].any(), "counters left non-zero or a bounded wait expired"


@pytest.mark.parametrize("T,x_seed", [(1, 0), (3, 1), (8, 2)])
def test_lowlat_fused_matches_oracle_and_the_five_launch_form(flint_bf16, attn_side, T, x_seed):
    say(f"low-latency path T={T} x_seed={x_seed}: fused and five-launch")
    a = run(flint_bf16, attn_side, T, x_seed, fused=True)
    check(flint_bf16, attn_side, a)
    b = run(flint_bf16, attn_side, T, x_seed, fused=False)
    for key in ("r1", "n", "ids", "w", "r_out", "n_out"):
        assert np.array_equal(a[key], b[key]), key
    assert not b["header"].any()


@pytest.mark.parametrize("T,x_seed", [(1, 0), (8, 2)])
def test_lowlat_nvfp4_fused_matches_oracle_and_the_five_launch_form(flint_nvfp4, attn_side, T,
                                                                     x_seed):
    """The same path over NVFP4 experts (the attention projection, router and
    norms stay bf16): tolerance 5e-2 x RMS of the layer part."""
    say(f"low-latency path, NVFP4 experts, T={T} x_seed={x_seed}: fused and five-launch")
    a = run(flint_nvfp4, attn_side, T, x_seed, fused=True)
    check(flint_nvfp4, attn_side, a)
    b = run(flint_nvfp4, attn_side, T, x_seed, fused=False)
    for key in ("r1", "n", "ids", "w", "r_out", "n_out"):
        assert np.array_equal(a[key], b[key]), key
    assert not b["header"].any()


def test_lowlat_without_next_norm_and_with_router_bias(flint_bf16, attn_side):
    say("low-latency path T=8, router bias, no next norm")
    r = run(flint_bf16, attn_side, 8, 3, fused=True, with_next=False, bias=True)
    assert r["n_out"] is None
    check(flint_bf16, attn_side, r, bias=True)


def test_lowlat_is_deterministic_and_repeatable(flint_bf16, attn_side):
    """Repeated fused forwards on one workspace (the counters must come back
    to zero every time) give the same bits."""
    say("low-latency path T=5, five forwards on one workspace")
    sg = flint_bf16["sg"]
    moe = sg.FlintMoE(max_tokens=8)
    T = 5
    d = lambda b: sg.bf16_tensor(b, "cuda")
    attn, rb = d(make_attn(T, seed=0, x_seed=9)), d(make_residual(T, seed=0, x_seed=9))
    gamma, gnext = d(flint_bf16["syn"].norm_weight()), d(attn_side["gnext"])
    ws = moe.new_workspace(T, "cuda")
    outs = []
    for _ in range(5):
        r_out = torch.empty((T, 2048), dtype=torch.bfloat16, device="cuda")
        n_out = torch.empty_like(r_out)
        moe.lowlat_forward(flint_bf16["W"], attn_side["wo_dev"], attn, rb, gamma, r_out,
                           gamma_next=gnext, n_out=n_out, eps=EPS, workspace=ws)
        outs.append((sg.bf16_bits(r_out), sg.bf16_bits(n_out)))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])
    assert not ws[:HDR_WORDS * 4].cpu().numpy().any()


def test_lowlat_rejects_batches_above_eight(flint_bf16, attn_side):
    sg = flint_bf16["sg"]
    moe = sg.FlintMoE(max_tokens=16)
    T = 9
    x = torch.zeros((T, 2048), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((T, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sg.FlintError) as e:
        moe.lowlat_forward(flint_bf16["W"], attn_side["wo_dev"], a, x, x[0], torch.empty_like(x))
    assert e.value.status == sg.FLINT_ERR_UNSUPPORTED

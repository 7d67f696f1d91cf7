"""GPU parity of the dense MLP (Flint's layers 0 and 1) against the fp64
oracle, through the C ABI: GEMV kernels for T <= 64, MFMA GEMMs above, bare
and as the pre-norm block.

Tolerances: max |out - oracle| <= 2e-2 * RMS(oracle MLP output) (+ 2^-8 |out|
for the block, whose sum with r is rounded once to bf16), the layer's bf16
bound; h (fp32 on the decode path) within 1e-4 of max |h| per token.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bf16_to_f64  # noqa: E402
from oracle.dense import DenseMLP, mlp_block_forward, mlp_forward  # noqa: E402
from oracle.grouped import mlp_forward_batched  # noqa: E402
from synth import SyntheticDenseMLP, make_residual, make_x  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-2
EPS = 1e-6
FLINT_INTER_D = 14336


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


_cache = {}


def dense(inter):
    """(synthetic weights, device tensors, oracle) for one intermediate size."""
    if inter not in _cache:
        if not torch.cuda.is_available():
            pytest.skip("no GPU")
        import sparse_expert_gemv_amd as sg
        say(f"generating dense MLP weights, I_d={inter}")
        S = SyntheticDenseMLP(seed=0, inter=inter)
        d = dict(sg=sg, S=S, w13=sg.bf16_tensor(S.w13(), "cuda"), w2=sg.bf16_tensor(S.w2(), "cuda"),
                 gamma=sg.bf16_tensor(S.norm_weight(), "cuda"),
                 M=DenseMLP(2048, inter, S.w13(), S.w2()))
        _cache.clear()          # keep one size resident at a time
        _cache[inter] = d
    return _cache[inter]


def run(d, xb, block=False, max_tokens=64):
    sg = d["sg"]
    T = xb.shape[0]
    m = sg.FlintMLP(inter=d["M"].inter, max_tokens=max_tokens)
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    ws = m.new_workspace(T, "cuda")
    m.forward(d["w13"], d["w2"], x, out, gamma=d["gamma"] if block else None, eps=EPS, workspace=ws)
    torch.cuda.synchronize()
    return sg.bf16_bits(out), ws, m.workspace_layout(T)


def check_out(out_bits, refs, block):
    got = bf16_to_f64(out_bits).reshape(out_bits.shape)
    ref = np.stack([r.out if block else r[0] for r in refs])
    mlp = np.stack([r.mlp_out if block else r[0] for r in refs])
    rms = float(np.sqrt(np.mean(mlp ** 2)))
    excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) if block else 0.0)
    ratio = float(max(0.0, np.max(excess))) / rms
    print(f"max excess / RMS(MLP out) = {ratio:.5f} (tol {TOL})")
    assert ratio <= TOL


@pytest.mark.parametrize("T,x_seed", [(1, 0), (8, 0), (13, 1), (64, 2)])
def test_dense_decode_matches_oracle(T, x_seed):
    d = dense(FLINT_INTER_D)
    say(f"dense decode parity I_d={FLINT_INTER_D} T={T}")
    xb = make_x(T, seed=0, x_seed=x_seed)
    out, ws, lay = run(d, xb)
    refs = mlp_forward(d["M"], xb)
    check_out(out, refs, block=False)
    h = ws[lay["h"]:lay["h"] + T * FLINT_INTER_D * 4].cpu().numpy().view(np.float32)
    h = h.reshape(T, FLINT_INTER_D)
    for t, (_, href) in enumerate(refs):
        np.testing.assert_allclose(h[t], href, rtol=0, atol=1e-4 * np.max(np.abs(href)))


@pytest.mark.parametrize("T,x_seed", [(1, 3), (8, 4)])
def test_dense_block_decode_matches_oracle(T, x_seed):
    d = dense(FLINT_INTER_D)
    say(f"dense block decode parity T={T}")
    rb = make_residual(T, seed=0, x_seed=x_seed)
    out, _, _ = run(d, rb, block=True)
    check_out(out, mlp_block_forward(d["M"], rb, d["S"].norm_weight(), EPS), block=True)


@pytest.mark.parametrize("T,block", [(65, False), (200, True)])
def test_dense_prefill_matches_oracle(T, block):
    d = dense(FLINT_INTER_D)
    say(f"dense prefill parity T={T} block={block}")
    xb = (make_residual if block else make_x)(T, seed=0, x_seed=5)
    out, _, _ = run(d, xb, block=block, max_tokens=8192)
    refs = (mlp_block_forward(d["M"], xb, d["S"].norm_weight(), EPS) if block
            else mlp_forward(d["M"], xb))
    check_out(out, refs, block)


def check_out_arrays(out_bits, ref, mlp, block):
    got = bf16_to_f64(out_bits).reshape(out_bits.shape)
    rms = float(np.sqrt(np.mean(mlp ** 2)))
    excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) if block else 0.0)
    ratio = float(max(0.0, np.max(excess))) / rms
    print(f"max excess / RMS(MLP out) = {ratio:.5f} (tol {TOL}) over {got.shape[0]} tokens")
    assert ratio <= TOL


@pytest.mark.parametrize("block", [False, True])
def test_dense_prefill_t8192_full(block):
    """Every token of a prefill-sized batch against the batched oracle."""
    d = dense(FLINT_INTER_D)
    T = 8192
    say(f"dense prefill T=8192 block={block}, every token")
    xb = (make_residual if block else make_x)(T, seed=0, x_seed=6)
    out, _, _ = run(d, xb, block=block, max_tokens=T)
    S = d["S"]
    if block:
        ref, mlp = mlp_forward_batched(S.w13(), S.w2(), xb, 2048, FLINT_INTER_D,
                                       gamma_bits=S.norm_weight(), eps=EPS)
    else:
        ref = mlp = mlp_forward_batched(S.w13(), S.w2(), xb, 2048, FLINT_INTER_D)
    check_out_arrays(out, ref, mlp, block)


@pytest.mark.parametrize("inter,T", [(512, 5), (1536, 3), (1536, 130)])
def test_dense_other_widths(inter, T):
    """Widths with fewer 512-column chunks than the down kernel has waves
    (one and three), on both paths."""
    d = dense(inter)
    say(f"dense I_d={inter} T={T}")
    xb = make_x(T, seed=0, x_seed=7)
    out, _, _ = run(d, xb, max_tokens=256)
    check_out(out, mlp_forward(d["M"], xb), block=False)


def test_dense_bitwise_deterministic():
    d = dense(1536)
    say("dense determinism T=8 and T=100")
    for T in (8, 100):
        xb = make_x(T, seed=0, x_seed=8)
        a, _, _ = run(d, xb, max_tokens=128)
        b, _, _ = run(d, xb, max_tokens=128)
        assert np.array_equal(a, b)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_dense_prefill_large_activations_past_fp16_range():
    """The dense MLP's gate/up weights times 2^8 (exact in bf16): |h| far past
    fp16's 65504 on the prefill path, every token against the oracle."""
    import sparse_expert_gemv_amd as sg
    from oracle.block import f64_to_bf16_bits
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("dense prefill with |h| past the fp16 range, I_d=512, T=130")
    S = SyntheticDenseMLP(seed=2, inter=512)
    w13 = f64_to_bf16_bits(bf16_to_f64(S.w13()) * 256.0).reshape(S.w13().shape)
    M = DenseMLP(2048, 512, w13, S.w2())
    xb = make_x(130, seed=2, x_seed=1)
    m = sg.FlintMLP(inter=512, max_tokens=256)
    x = sg.bf16_tensor(xb, "cuda")
    out = torch.empty_like(x)
    m.forward(sg.bf16_tensor(w13, "cuda"), sg.bf16_tensor(S.w2(), "cuda"), x, out)
    torch.cuda.synchronize()
    refs = mlp_forward(M, xb)
    h_max = max(float(np.max(np.abs(h))) for _, h in refs)
    print(f"max |h| = {h_max:.3e}")
    assert h_max > 4 * 65504
    check_out(sg.bf16_bits(out), refs, block=False)

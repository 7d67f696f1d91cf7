"""GPU check of flint_moe_forward_noalloc (the forward whose workspace is the
library's static device scratch array) against flint_moe_forward with a
caller workspace: two calls in a row, the second with a smaller batch, each
bit-identical to the workspace forward (the same kernels run on the same
inputs) and within the bf16 tolerance of the fp64 oracle."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import moe_forward  # noqa: E402
from oracle.grading import TOL_BF16, grade  # noqa: E402
from synth import make_x  # noqa: E402

pytestmark = pytest.mark.gpu


def test_noalloc_forward_matches_workspace_forward(flint_bf16):
    dev = flint_bf16
    sg = dev["sg"]
    moe = sg.FlintMoE(max_tokens=64)
    # T = 16 runs the 16-wave router with the ticketed routing block; T = 3
    # the small-batch path whose gate/up blocks route the batch themselves.
    for T, x_seed in ((16, 21), (3, 22)):
        print(f"[gpu-case] no-alloc forward T={T} x_seed={x_seed}", flush=True)
        xb = make_x(T, seed=0, x_seed=x_seed)
        x = sg.bf16_tensor(xb, "cuda")
        res = []
        for noalloc in (False, True):
            out = torch.empty_like(x)
            ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
            w = torch.zeros((T, 6), dtype=torch.float32, device="cuda")
            if noalloc:
                moe.forward_noalloc(dev["W"], x, out, ids, w)
            else:
                moe.forward(dev["W"], x, out, ids, w, moe.new_workspace(T, "cuda"))
            torch.cuda.synchronize()
            res.append((sg.bf16_bits(out), ids.cpu().numpy(), w.cpu().numpy()))
        (o0, i0, w0), (o1, i1, w1) = res
        assert np.array_equal(o0, o1)
        assert np.array_equal(i0, i1)
        assert np.array_equal(w0, w1)
        g = grade(o1, i1, moe_forward(dev["L"], xb), tol=TOL_BF16)
        print(g)
        assert g.ok, str(g)


def test_noalloc_rejects_batches_beyond_its_scratch(flint_bf16):
    sg = flint_bf16["sg"]
    moe = sg.FlintMoE(max_tokens=128)
    x = torch.zeros((65, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sg.FlintError) as e:
        moe.forward_noalloc(flint_bf16["W"], x, torch.empty_like(x))
    assert e.value.status == sg.FLINT_ERR_UNSUPPORTED
    assert "T <= 64" in moe.last_error()

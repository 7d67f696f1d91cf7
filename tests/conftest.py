"""Shared pytest configuration: the ``gpu`` marker and repository import path."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def flint_bf16():
    """The seeded full-size bf16 layer on cuda:0, with its oracle (GPU tests only)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_expert_gemv_amd as sg
    from oracle import OracleLayer
    from synth import SyntheticLayer
    from synth.device import upload_bf16
    print("[gpu-case] generating seeded layer 0", flush=True)
    syn = SyntheticLayer(0)
    syn.routed_banks()
    t = upload_bf16(syn, "cuda", with_bias=True)
    bank = sg.DeviceBank(t["w13"], t["w2"])
    shared = sg.DeviceBank(t["sh_w13"], t["sh_w2"])
    return dict(
        sg=sg, syn=syn, t=t,
        W=sg.DeviceWeights(t["router_w"], None, bank, shared),
        Wb=sg.DeviceWeights(t["router_w"], t["router_b"], bank, shared),
        L=OracleLayer(2048, 256, 6, 512, syn.router_w(), None, syn.expert),
        Lb=OracleLayer(2048, 256, 6, 512, syn.router_w(), syn.router_bias(), syn.expert))


@pytest.fixture(scope="session")
def flint_nvfp4():
    """The seeded layer encoded as NVFP4 on cuda:0, with its oracles (GPU tests only):
    L / Lb evaluate the decoded NVFP4 weights, L16 the bf16 weights they encode."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_expert_gemv_amd as sg
    from oracle import OracleLayer
    from synth import SyntheticLayer
    from synth.device import nvfp4_layer, upload_nvfp4
    print("[gpu-case] generating and encoding the NVFP4 layer", flush=True)
    syn = SyntheticLayer(0)
    syn.routed_banks()
    q = nvfp4_layer(syn)
    t = upload_nvfp4(syn, q, "cuda", with_bias=True)

    def bank(name):
        return sg.DeviceBank(t[f"{name}_w13_q"], t[f"{name}_w2_q"], t[f"{name}_w13_s"],
                             t[f"{name}_w2_s"], t[f"{name}_w13_g"], t[f"{name}_w2_g"])

    def raw(e):
        b, i = ("shared", 0) if e < 0 else ("routed", e)
        d = q[b]
        return ((d["w13_q"][i], d["w13_s"][i], d["w13_g"][i]),
                (d["w2_q"][i], d["w2_s"][i], d["w2_g"][i]))

    return dict(
        sg=sg, syn=syn, t=t, fmt=sg.FLINT_W_NVFP4,
        W=sg.DeviceWeights(t["router_w"], None, bank("routed"), bank("shared")),
        Wb=sg.DeviceWeights(t["router_w"], t["router_b"], bank("routed"), bank("shared")),
        L=OracleLayer(2048, 256, 6, 512, syn.router_w(), None, raw, fmt="nvfp4"),
        Lb=OracleLayer(2048, 256, 6, 512, syn.router_w(), syn.router_bias(), raw, fmt="nvfp4"),
        L16=OracleLayer(2048, 256, 6, 512, syn.router_w(), None, syn.expert))

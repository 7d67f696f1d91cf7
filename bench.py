#!/usr/bin/env python3
"""Benchmark of the Flint MoE feed-forward layer on one MI355X.

One step = one whole layer forward (router GEMV, sigmoid top-6, bucketing,
gate/up GEMV with SiLU-and-mul, down GEMV with the weighted combine) over one
batch of T tokens, through the C ABI, on the seeded synthetic layer.

The default run measures every configuration the metric is quoted on, in one
process: decode T=1, T=8 (the headline `value`) and T=32 with skewed routing
(bf16), NVFP4 weights at T=1 and T=8, and the T=8192 prefill.  Each lands in
`per_config` with its µs per layer, tokens/s, the layer's algorithmic GB/s
and fraction of the 8 TB/s HBM peak, its per-kernel times and the roofline of
its dominant launch.  The low-latency decode path (attention output
projection, residual, norms and the layer; three launches and five) is measured
at T=1 and T=8 over bf16 and over NVFP4 experts.  `--workload NAME` measures
one configuration alone.

To measure HBM rather than the 256 MB Infinity Cache, the layer is cloned
into several device copies and step i runs on copy i mod copies.  The K
timed steps are captured in one HIP graph and replayed once, bracketed by
synchronisation and HIP events on the replay stream.  Per-kernel durations
come from a separate eager pass of K steps in which each kernel is launched
with a start and a stop event that take its own execution timestamps
(flint_moe_forward_timed).

`hbm_calibration` is the read rate of a plain coalesced streaming kernel
(flint_moe_calib_stream_read) over buffers of the T=1 and T=8 layers' sizes
and over 4 GiB, each window read once per step from a rotating set so that
no step hits the Infinity Cache: what is achievable, beside the nominal peak.

The roofline's "traffic" (HBM bytes per launch of the dominant kernel) is
read from the counter table in profiles/hbm_traffic.md when its row was
measured on the kernel sources as they are now (SHA-256 of the path's .hip
file and the two shared headers); otherwise it is null.  "traffic_GBps" is
that byte count over the launch's measured average duration.

`cpu_baseline` times the oracle (fp64 NumPy, as it stands) on the host on the
same tokens: the bf16 -> fp64 weight conversion is done once before the timed
runs, and each configuration is timed with the BLAS library on every core of
the process's affinity mask and on one thread (median of 3 runs; the prefill
batch: one run, on every core only).

With --block, one step is the pre-norm block around the layer instead
(flint_moe_block_forward: RMSNorm of the residual stream r, the layer, and
the residual add), on a synthetic residual stream and norm gain.  With
--mlp, one step is the dense SwiGLU MLP of Flint's first two layers
(flint_mlp_forward; intermediate size --mlp-inter), bare or with --block.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

METRIC = "µs per MoE layer forward at T=1/8/32 + achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
H, E, K_TOP, I = 2048, 256, 6, 512
ROUTER_BYTES = E * H * 2                   # 1,048,576
# Algorithmic bytes of one expert's gate/up and down weights.
EXPERT_BYTES = {
    "bf16": (2 * I * H * 2, H * I * 2),                               # 4,194,304 + 2,097,152
    "nvfp4": (2 * I * H // 2 + 2 * I * H // 16 + 4, H * I // 2 + H * I // 16 + 4),  # 1,179,652 + 589,828
}

WORKLOADS = {
    "decode_t1": dict(T=1, bias=False, fmt="bf16"),
    "decode_t8": dict(T=8, bias=False, fmt="bf16"),
    "decode_t32_skewed": dict(T=32, bias=True, fmt="bf16"),
    "decode_nvfp4_t1": dict(T=1, bias=False, fmt="nvfp4"),
    "decode_nvfp4_t8": dict(T=8, bias=False, fmt="nvfp4"),
    "prefill_t8192": dict(T=8192, bias=False, fmt="bf16"),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0
EPS = 1e-6                                 # RMSNorm eps of the pre-norm block


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "sparse_expert_gemv_amd", "csrc")
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def kernel_sources_sha(path_file: str) -> str:
    """SHA-256 (first 16 hex digits) over a path's kernel source and the shared headers."""
    h = hashlib.sha256()
    for f in (path_file, "flint_device.h", "flint_kernels.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str, sha: str):
    """HBM bytes per launch from the counter table, or None if absent or stale.

    Table rows: | workload | kernel | sources sha | FETCH KiB | WRITE KiB | bytes |"""
    try:
        with open(TRAFFIC_TABLE) as fh:
            for line in fh:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                if len(cells) >= 6 and cells[0] == workload and cells[1] == kernel:
                    if cells[2] == sha and re.fullmatch(r"\d+", cells[5]):
                        return int(cells[5])
    except OSError:
        pass
    return None


def with_traffic_rate(roof: dict) -> dict:
    """Adds the counter-measured HBM rate of the dominant launch: its
    FETCH_SIZE + WRITE_SIZE bytes per launch over its average launch time."""
    t = roof.get("traffic")
    roof["traffic_GBps"] = round(t / (roof["avg_launch_us"] * 1e-6) / 1e9, 1) if t else None
    return roof


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="suite", choices=["suite"] + sorted(WORKLOADS),
                   help="suite (default): every configuration, T=8 bf16 as the headline")
    p.add_argument("--copies", type=int, default=0,
                   help="device copies of the layer (0: 32, or 8 for --workload prefill_t8192)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                   help="CPU time budget of the oracle baseline in --mlp runs (0 disables the "
                        "baseline in every mode)")
    p.add_argument("--block", action="store_true",
                   help="time the pre-norm block (RMSNorm + layer + residual add)")
    p.add_argument("--mlp", action="store_true",
                   help="time the dense MLP of layers 0-1 instead of the MoE layer")
    p.add_argument("--lowlat", action="store_true",
                   help="also time the low-latency decode path (attention output projection, "
                        "layer, next norm) at T=1 and T=8, fused and in five launches")
    p.add_argument("--mlp-inter", type=int, default=14336,
                   help="intermediate size of the dense MLP")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run a device copy of this many MiB (FETCH_SIZE calibration)")
    return p.parse_args()


def blas_threads() -> int:
    """Threads the BLAS library behind numpy actually uses."""
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()
                    if d.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def blas_info() -> str:
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                return (f"{d.get('internal_api')} {d.get('version')} "
                        f"({d.get('threading_layer')}, {d.get('num_threads')} threads)")
    except Exception:
        pass
    return "unknown"


def oracle_layer(syn, fmt, bias, nvq=None):
    """The oracle's view of the seeded layer (for nvfp4: the NVFP4 encoding of
    the same tensors, which the oracle decodes)."""
    from oracle import OracleLayer
    from synth.device import nvfp4_layer
    if fmt == "bf16":
        raw = syn.expert
    else:
        q = nvq if nvq is not None else nvfp4_layer(syn)

        def raw(e):
            bank, i = (q["shared"], 0) if e < 0 else (q["routed"], e)
            return ((bank["w13_q"][i], bank["w13_s"][i], float(bank["w13_g"][i])),
                    (bank["w2_q"][i], bank["w2_s"][i], float(bank["w2_g"][i])))
    return OracleLayer(H, E, K_TOP, I, syn.router_w(), syn.router_bias() if bias else None, raw,
                       fmt=fmt)


def time_oracle(fn, runs):
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    times.sort()
    return times[len(times) // 2]


def cpu_oracle_config(layer, x_bits, block_gamma=None, prefill=False):
    """The oracle on one configuration's tokens: per-token loop (decode) or the
    expert-grouped evaluation (prefill), every core and one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import moe_token
    from oracle.block import block_token
    from oracle.grouped import block_forward_grouped, moe_forward_grouped
    T = x_bits.shape[0]
    cores = len(os.sched_getaffinity(0))
    if prefill:
        cache = {e: layer.expert_f64(e) for e in range(-1, E)}
        layer.expert_f64 = cache.__getitem__          # conversion done: outside the timed run
        layer.router_f64()
        if block_gamma is None:
            fn = lambda: moe_forward_grouped(layer, x_bits)
        else:
            fn = lambda: block_forward_grouped(layer, x_bits, block_gamma)
        with threadpool_limits(limits=cores, user_api="blas"):
            threads = blas_threads()
            t_all = time_oracle(fn, 1)
        del layer.expert_f64
        return {"us_per_layer": round(t_all * 1e6, 1), "tokens_per_s": round(T / t_all, 1),
                "us_per_layer_1thread": None, "runs": 1, "blas_threads": threads,
                "form": "expert-grouped fp64 (oracle.grouped), one run on every core; "
                        "one thread not timed (several minutes)"}
    cache: dict = {}
    if block_gamma is None:
        fn = lambda: [moe_token(layer, x_bits[t], expert_cache=cache) for t in range(T)]
    else:
        fn = lambda: [block_token(layer, x_bits[t], block_gamma, expert_cache=cache)
                      for t in range(T)]
    fn()                                              # fills the fp64 expert cache, untimed
    with threadpool_limits(limits=cores, user_api="blas"):
        threads = blas_threads()
        t_all = time_oracle(fn, 3)
    with threadpool_limits(limits=1, user_api="blas"):
        t_one = time_oracle(fn, 3)
    return {"us_per_layer": round(t_all * 1e6, 1), "tokens_per_s": round(T / t_all, 1),
            "us_per_layer_1thread": round(t_one * 1e6, 1), "runs": 3, "blas_threads": threads,
            "form": "per-token fp64 loop (oracle.moe_token), median of 3"}


def kernel_names(nk: int, mlp: bool):
    if mlp:
        return {2: ["gateup", "down"], 3: ["norm", "gateup", "down"]}.get(
            nk, [f"kernel{i}" for i in range(nk)])
    return {3: ["route", "gateup", "down"],
            5: ["router", "bucket", "gateup", "down", "shared_down_combine"],
            6: ["norm", "router", "bucket", "gateup", "down", "shared_down_combine"]}.get(
                nk, [f"kernel{i}" for i in range(nk)])


def time_kernels(timed_step, steps, stream, mlp=False, names=None):
    """K eager steps, each kernel bracketed by its own start/stop events.
    Returns (names, mean us per kernel, eager wall us per step)."""
    import numpy as np
    import torch
    n_ev = 16
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    nk = 0
    t0 = time.perf_counter()
    for i in range(steps):
        nk = timed_step(i, stream.cuda_stream, [e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    eager_wall = (time.perf_counter() - t0) / steps
    kern_ms = np.array([[evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for j in range(nk)]
                        for i in range(steps)])
    names = names[:nk] if names else kernel_names(nk, mlp)
    kern_us = kern_ms.mean(axis=0) * 1e3
    log("per-kernel us: " + ", ".join(f"{n}={v:.2f}" for n, v in zip(names, kern_us)))
    return names, kern_us, eager_wall * 1e6


def time_graph(step, steps, dev):
    """The timed region: one HIP-graph replay of exactly K steps between events
    on the replay stream.  Returns us per step."""
    import torch
    stream = torch.cuda.current_stream(dev)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(0, side.cuda_stream)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream(dev).cuda_stream
        for i in range(steps):
            step(i, cap)
    torch.cuda.synchronize()
    g.replay()                       # upload + first launch, untimed
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1e3 / steps
    log(f"graph: {us_step:.2f} us/step over {steps} steps")
    return us_step


def calibration_copy(args, dev):
    import torch
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * 2**20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")


def common_result(args, us_step, dtype, config):
    return {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": config,
    }


def run_mlp(args, rank):
    """The dense MLP of layers 0 and 1 (bare, or the pre-norm block)."""
    import torch

    import sparse_expert_gemv_amd as sg
    from synth import SyntheticDenseMLP, make_residual, make_x

    wl = WORKLOADS[args.workload]
    T, Id = wl["T"], args.mlp_inter
    if wl["fmt"] != "bf16" or wl["bias"]:
        raise SystemExit("--mlp takes the bf16 workloads without router bias "
                         "(decode_t1, decode_t8, prefill_t8192)")
    if args.copies <= 0:
        args.copies = 8 if T <= 64 else 4
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"dense MLP I_d={Id}, workload {args.workload}: generating seeded weights {args.seed}")
    S = SyntheticDenseMLP(args.seed, Id)
    w13 = [sg.bf16_tensor(S.w13(), dev)]
    w2 = [sg.bf16_tensor(S.w2(), dev)]
    for _ in range(1, args.copies):
        w13.append(w13[0].clone())
        w2.append(w2[0].clone())
    torch.cuda.synchronize()
    log(f"{args.copies} weight copies resident ({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    m = sg.FlintMLP(inter=Id, max_tokens=max(T, 1))
    x_bits = (make_residual if args.block else make_x)(T, seed=args.seed, x_seed=0)
    x = sg.bf16_tensor(x_bits, dev)
    gamma = sg.bf16_tensor(S.norm_weight(), dev)
    out = torch.empty_like(x)
    ws = m.new_workspace(T, dev)
    gp = int(gamma.data_ptr()) if args.block else None
    wp = [(int(a.data_ptr()), int(b.data_ptr())) for a, b in zip(w13, w2)]
    xp, op, wsp, wsb = int(x.data_ptr()), int(out.data_ptr()), int(ws.data_ptr()), ws.numel()

    def step(i, sh):
        a, b = wp[i % len(wp)]
        st = m.forward_raw(a, b, gp, EPS, xp, T, op, wsp, wsb, sh)
        if st != sg.FLINT_OK:
            raise sg.FlintError(st, m.last_error())

    def timed_step(i, sh, events):
        a, b = wp[i % len(wp)]
        st, nk = m.forward_timed_raw(a, b, gp, EPS, xp, T, op, wsp, wsb, sh, events)
        if st != sg.FLINT_OK:
            raise sg.FlintError(st, m.last_error())
        return nk

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()
    names, kern_us, eager_us = time_kernels(timed_step, args.steps, stream, mlp=True)
    us_step = time_graph(step, args.steps, dev)

    w13_bytes, w2_bytes = 2 * Id * H * 2, H * Id * 2
    layer_bytes = w13_bytes + w2_bytes + 2 * T * H * 2 + (H * 2 if args.block else 0)
    flops = 2.0 * T * 3 * Id * H
    sha = kernel_sources_sha("decode.hip" if T <= 64 else "prefill.hip")
    wl_name = "mlp_" + ("block_" if args.block else "") + args.workload
    gi = names.index("gateup")
    dom_us = float(kern_us[gi])
    if T <= 64:
        achieved = w13_bytes / (dom_us * 1e-6) / 1e9
        roof = {"kernel": "gateup", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(wl_name, "gateup", sha),
                "algorithmic_bytes_per_launch": w13_bytes, "avg_launch_us": round(dom_us, 3)}
    else:
        gu_flops = 2.0 * T * 2 * Id * H
        achieved = gu_flops / (dom_us * 1e-6) / 1e12
        roof = {"kernel": "gateup", "bound": "mfma", "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(wl_name, "gateup", sha),
                "algorithmic_flops_per_launch": gu_flops, "avg_launch_us": round(dom_us, 3)}
    calibration_copy(args, dev)
    config = {"workload": f"flint_dense_{wl_name}", "T": T, "hidden": H, "inter": Id,
              "seed": args.seed, "weight_copies": args.copies,
              "timing": "one HIP-graph replay of K steps",
              **({"prenorm_block": {"norm": "RMSNorm", "eps": EPS, "residual_add": True}}
                 if args.block else {})}
    result = common_result(args, us_step, "bf16", config)
    result.update({
        "tokens_per_s": round(T / (us_step * 1e-6), 1),
        "layer_algorithmic_bytes": layer_bytes,
        "layer_GBps": round(layer_bytes / (us_step * 1e-6) / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "layer_algorithmic_flops": flops,
        "kernels_us": {n: round(float(v), 3) for n, v in zip(names, kern_us)},
        "kernel_timing": "start/stop timestamps of each kernel's execution (hipExtLaunchKernelGGL "
                         "events), averaged over K eager steps",
        "eager_wall_us_per_step": round(eager_us, 2),
        "roofline": with_traffic_rate(roof),
    })
    if rank == 0 and args.cpu_baseline_seconds > 0:
        log("timing the oracle on the host")
        result["cpu_baseline"] = mlp_cpu_baseline(S, x_bits, args.block, args.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)


def mlp_cpu_baseline(S, x_bits, block, budget_s):
    """The dense-MLP oracle, as it stands, on the same tokens (at least two runs)."""
    from oracle.dense import DenseMLP, mlp_block_forward, mlp_forward
    threads = blas_threads()
    M = DenseMLP(H, S.inter, S.w13(), S.w2())
    times = []
    t_end = time.perf_counter() + budget_s
    while len(times) < 2 or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        if block:
            mlp_block_forward(M, x_bits, S.norm_weight())
        else:
            mlp_forward(M, x_bits)
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    T = x_bits.shape[0]
    return {"value": med * 1e6, "unit": "us/layer", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} whole-MLP forwards of the same {T} tokens "
                      f"(fp64 numpy, per-token loop); median",
            "tokens_per_s": T / med}


SUITE = ("decode_t1", "decode_t8", "decode_t32_skewed", "decode_nvfp4_t1", "decode_nvfp4_t8",
         "prefill_t8192")
HEADLINE = "decode_t8"
# Spec target: bf16 decode at T=1 and T=8 sustains >= 70% of the HBM peak
# on the selected experts' bytes.
TARGET_FRAC = {"decode_t1": 0.70, "decode_t8": 0.70}


def upload_copies(syn, fmt, n_copies, dev, nvq=None):
    """n_copies device copies of the seeded layer (weights only; one bias
    tensor, shared).  Returns a list of tensor dicts."""
    import torch
    from synth.device import upload_bf16, upload_nvfp4
    base = (upload_bf16(syn, dev, with_bias=True) if fmt == "bf16"
            else upload_nvfp4(syn, nvq, dev, with_bias=True))
    copies = [base]
    for _ in range(1, n_copies):
        copies.append({k: (v if k == "router_b" else v.clone()) for k, v in base.items()})
    torch.cuda.synchronize()
    return copies


def weight_structs(sg, copies, fmt, bias):
    out = []
    for t in copies:
        if fmt == "bf16":
            routed = sg.DeviceBank(t["w13"], t["w2"])
            shared = sg.DeviceBank(t["sh_w13"], t["sh_w2"])
        else:
            routed, shared = (sg.DeviceBank(t[f"{n}_w13_q"], t[f"{n}_w2_q"], t[f"{n}_w13_s"],
                                            t[f"{n}_w2_s"], t[f"{n}_w13_g"], t[f"{n}_w2_g"])
                              for n in ("routed", "shared"))
        out.append(sg.DeviceWeights(t["router_w"], t["router_b"] if bias else None, routed,
                                    shared).struct())
    return out


def measure(args, name, structs, dev, gamma, x_bits):
    """Times one configuration; returns its per-config entry."""
    import numpy as np
    import torch

    import sparse_expert_gemv_amd as sg

    wl = WORKLOADS[name]
    T, fmt = wl["T"], wl["fmt"]
    moe = sg.FlintMoE(max_tokens=max(T, 1),
                      fmt=sg.FLINT_W_BF16 if fmt == "bf16" else sg.FLINT_W_NVFP4)
    x = sg.bf16_tensor(x_bits, dev)
    out = torch.empty_like(x)
    ids = torch.empty((T, K_TOP), dtype=torch.int32, device=dev)
    wts = torch.empty((T, K_TOP), dtype=torch.float32, device=dev)
    ws = moe.new_workspace(T, dev)
    ws_bytes = ws.numel()
    gamma_ptr = int(gamma.data_ptr())
    ptrs = (int(x.data_ptr()), int(out.data_ptr()), int(ids.data_ptr()), int(wts.data_ptr()),
            int(ws.data_ptr()))

    def step(i, sh):
        if args.block:
            st = moe.block_forward_raw(structs[i % len(structs)], gamma_ptr, EPS, ptrs[0], T,
                                       ptrs[1], ptrs[2], ptrs[3], ptrs[4], ws_bytes, sh)
        else:
            st = moe.forward_raw(structs[i % len(structs)], ptrs[0], T, ptrs[1], ptrs[2], ptrs[3],
                                 ptrs[4], ws_bytes, sh)
        if st != sg.FLINT_OK:
            raise sg.FlintError(st, moe.last_error())

    def timed(i, sh, events):
        if args.block:
            st, nk = moe.block_forward_timed_raw(structs[i % len(structs)], gamma_ptr, EPS,
                                                 ptrs[0], T, ptrs[1], ptrs[2], ptrs[3], ptrs[4],
                                                 ws_bytes, sh, events)
        else:
            st, nk = moe.forward_timed_raw(structs[i % len(structs)], ptrs[0], T, ptrs[1],
                                           ptrs[2], ptrs[3], ptrs[4], ws_bytes, sh, events)
        if st != sg.FLINT_OK:
            raise sg.FlintError(st, moe.last_error())
        return nk

    log(f"{name}: warm-up")
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()
    n_active = int(np.unique(ids.cpu().numpy()).size)
    log(f"{name}: |U| = {n_active}")
    names, kern_us, eager_us = time_kernels(timed, args.steps, stream)
    us_step = time_graph(step, args.steps, dev)

    sha = kernel_sources_sha("decode.hip" if T <= 64 else "prefill.hip")
    wl_name = ("block_" if args.block else "") + name
    w13_bytes, w2_bytes = EXPERT_BYTES[fmt]
    # Weights read once, the input read once, the output written once (+ the
    # norm gain for the block).
    layer_bytes = ROUTER_BYTES + (n_active + 1) * (w13_bytes + w2_bytes) + 2 * T * H * 2
    if args.block:
        layer_bytes += H * 2
    layer_flops = 2.0 * T * E * H + 2.0 * T * (K_TOP + 1) * 3 * I * H
    gi = names.index("gateup")
    dom_us = float(kern_us[gi])
    if T <= 64:
        # Dominant kernel: the gate/up GEMV launch, which streams the gate/up
        # weights of the |U| selected experts and of the shared expert.
        dom_bytes = (n_active + 1) * w13_bytes
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        roof = {"kernel": "gateup", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(wl_name, "gateup", sha),
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3)}
    else:
        # Dominant kernel: the grouped gate/up GEMM, 2 * (T * 7) * 1024 * 2048 flops.
        flops = 2.0 * T * (K_TOP + 1) * (2 * I) * H
        achieved = flops / (dom_us * 1e-6) / 1e12
        roof = {"kernel": "gateup", "bound": "mfma", "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(wl_name, "gateup", sha),
                "algorithmic_flops_per_launch": flops, "avg_launch_us": round(dom_us, 3)}
    layer_gbps = layer_bytes / (us_step * 1e-6) / 1e9
    entry = {
        "workload": f"flint_moe_{wl_name}", "T": T, "weights": fmt,
        "router_bias": wl["bias"], "n_active": n_active,
        "us_per_layer": round(us_step, 3),
        "tokens_per_s": round(T / (us_step * 1e-6), 1),
        "layer_algorithmic_bytes": layer_bytes,
        "layer_GBps": round(layer_gbps, 1),
        "layer_hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "layer_algorithmic_flops": layer_flops,
        "kernels_us": {n: round(float(v), 3) for n, v in zip(names, kern_us)},
        "eager_wall_us_per_step": round(eager_us, 2),
        "roofline": with_traffic_rate(roof),
    }
    if T > 64:
        tf = layer_flops / (us_step * 1e-6) / 1e12
        entry["layer_TFLOPs"] = round(tf, 1)
        entry["layer_mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
    if name in TARGET_FRAC and not args.block:
        tgt_us = layer_bytes / (TARGET_FRAC[name] * HBM_PEAK_GBPS * 1e9) * 1e6
        entry["target"] = {"layer_hbm_frac": TARGET_FRAC[name], "us_per_layer": round(tgt_us, 2),
                           "met": bool(layer_gbps / HBM_PEAK_GBPS >= TARGET_FRAC[name])}
    log(f"{name}: {us_step:.2f} us/layer, {layer_gbps:.0f} GB/s "
        f"({100 * layer_gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
    return entry


LOWLAT_NAMES = {True: ["oproj_route", "gateup", "down_nextnorm"],
                False: ["oproj", "route", "gateup", "down", "nextnorm"]}


def measure_lowlat(args, T, structs, wo_copies, dev, syn, fmt="bf16"):
    """The low-latency decode path (attention output projection + residual +
    norm + layer + residual + next norm) at T tokens, fused (three launches)
    and in five launches, over bf16 or NVFP4 experts; returns a per-config entry."""
    import numpy as np
    import torch

    import sparse_expert_gemv_amd as sg
    from synth import make_attn, make_next_gain, make_residual

    moe = sg.FlintMoE(max_tokens=8, fmt=sg.FLINT_W_NVFP4 if fmt == "nvfp4" else sg.FLINT_W_BF16)
    d = lambda b: sg.bf16_tensor(b, dev)
    attn = d(make_attn(T, seed=args.seed, x_seed=0))
    r = d(make_residual(T, seed=args.seed, x_seed=0))
    gamma, gnext = d(syn.norm_weight()), d(make_next_gain(seed=args.seed))
    r_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    n_out = torch.empty_like(r_out)
    ids = torch.empty((T, K_TOP), dtype=torch.int32, device=dev)
    ws = moe.new_workspace(T, dev)
    P = lambda t: int(t.data_ptr())
    wos = [P(w) for w in wo_copies]
    tag = "nvfp4_" if fmt == "nvfp4" else ""
    entry = {"workload": f"flint_moe_lowlat_{tag}t{T}", "T": T, "weights": fmt,
             "path": "r1 = r + Wo a; n = RMSNorm(r1) g; r_out = r1 + MoE(n); "
                     "n_out = RMSNorm(r_out) g_next"}
    stream = torch.cuda.current_stream(dev)
    for fused in (True, False):
        def step(i, sh, fused=fused):
            st = moe.lowlat_forward_raw(structs[i % len(structs)], wos[i % len(wos)], P(attn), P(r),
                                        P(gamma), P(gnext), EPS, T, P(r_out), P(n_out), P(ids), None,
                                        P(ws), ws.numel(), fused, sh)
            if st != sg.FLINT_OK:
                raise sg.FlintError(st, moe.last_error())

        def timed(i, sh, events, fused=fused):
            st, nk = moe.lowlat_forward_timed_raw(structs[i % len(structs)], wos[i % len(wos)],
                                                  P(attn), P(r), P(gamma), P(gnext), EPS, T,
                                                  P(r_out), P(n_out), P(ids), None, P(ws),
                                                  ws.numel(), fused, sh, events)
            if st != sg.FLINT_OK:
                raise sg.FlintError(st, moe.last_error())
            return nk

        for i in range(args.warmup):
            step(i, stream.cuda_stream)
        torch.cuda.synchronize()
        n_active = int(np.unique(ids.cpu().numpy()).size)
        names, kern_us, eager_us = time_kernels(timed, args.steps, stream, names=LOWLAT_NAMES[fused])
        us = time_graph(step, args.steps, dev)
        key = "fused" if fused else "unfused"
        entry[key] = {"launches": len(names), "us_per_step": round(us, 3),
                      "kernels_us": {n: round(float(v), 3) for n, v in zip(names, kern_us)},
                      "eager_wall_us_per_step": round(eager_us, 2)}
        entry["n_active"] = n_active
        log(f"lowlat {fmt} T={T} {key}: {us:.2f} us/step over {len(names)} launches")
    w13_bytes, w2_bytes = EXPERT_BYTES[fmt]
    entry["algorithmic_bytes"] = (H * 4096 * 2 + ROUTER_BYTES + (entry["n_active"] + 1) *
                                  (w13_bytes + w2_bytes) + T * (4096 + 4 * H) * 2 + 2 * H * 2)
    entry["fused_speedup"] = round(entry["unfused"]["us_per_step"] / entry["fused"]["us_per_step"], 3)
    return entry


def hbm_calibration(args, dev, sizes):
    """Read rate of the plain streaming kernel at each size (bytes): windows of
    that size from a 4 GiB buffer, a different window each step (the set is
    far larger than the Infinity Cache), K steps in one graph replay."""
    import torch

    import sparse_expert_gemv_amd as sg
    total = 4 * 2**30
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(sg.CALIB_SINK_WORDS, dtype=torch.int32, device=dev)
    base, sp = int(buf.data_ptr()), int(sink.data_ptr())
    out = {}
    for label, nbytes in sizes:
        nbytes = min(nbytes // 256 * 256, total)
        n_win = total // nbytes

        def step(i, sh, nbytes=nbytes, n_win=n_win):
            sg.calib_stream_read(base + (i % n_win) * nbytes, nbytes, sp, sh)

        steps = max(4, min(args.steps, 64)) if nbytes < total else 4
        us = time_graph(step, steps, dev)
        out[label] = {"bytes": nbytes, "us": round(us, 3),
                      "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        log(f"stream read {label}: {out[label]['GBps']} GB/s")
    del buf
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert parallelism across GPUs is not implemented). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))
    if args.mlp:
        if args.workload == "suite":
            args.workload = HEADLINE
        return run_mlp(args, rank)

    import torch

    import sparse_expert_gemv_amd as sg
    from synth import SyntheticLayer, make_residual, make_x
    from synth.device import nvfp4_layer

    names = list(SUITE) if args.workload == "suite" else [args.workload]
    headline = HEADLINE if args.workload == "suite" else args.workload
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copies <= 0:
        args.copies = 8 if names == ["prefill_t8192"] else 32

    log(f"generating seeded layer {args.seed}")
    syn = SyntheticLayer(args.seed)
    syn.routed_banks()
    gamma = sg.bf16_tensor(syn.norm_weight(), dev)
    make_in = make_residual if args.block else make_x
    inputs = {n: make_in(WORKLOADS[n]["T"], seed=args.seed, x_seed=0) for n in names}
    entries = {}
    nvq = None
    for fmt in ("bf16", "nvfp4"):
        todo = [n for n in names if WORKLOADS[n]["fmt"] == fmt]
        if not todo:
            continue
        if fmt == "nvfp4":
            log("encoding the layer as NVFP4")
            nvq = nvfp4_layer(syn)
        copies = upload_copies(syn, fmt, args.copies, dev, nvq)
        log(f"{fmt}: {args.copies} layer copies resident "
            f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")
        for n in todo:
            structs = weight_structs(sg, copies, fmt, WORKLOADS[n]["bias"])
            entries[n] = measure(args, n, structs, dev, gamma, inputs[n])
        if (args.workload == "suite" or args.lowlat) and not args.block:
            from synth import make_o_proj
            wo0 = sg.bf16_tensor(make_o_proj(seed=args.seed), dev)
            wo_copies = [wo0] + [wo0.clone() for _ in range(1, len(copies))]
            structs = weight_structs(sg, copies, fmt, False)
            tag = "nvfp4_" if fmt == "nvfp4" else ""
            for T in (1, 8):
                entries[f"lowlat_{tag}t{T}"] = measure_lowlat(args, T, structs, wo_copies, dev, syn,
                                                              fmt)
            del wo_copies, wo0
        del copies
        torch.cuda.empty_cache()

    calib = None
    if args.workload == "suite":
        calib = hbm_calibration(args, dev, [
            ("45MB", 45_096_960), ("284MB", 284_229_632), ("4GiB", 4 * 2**30)])
    calibration_copy(args, dev)

    cpu = None
    if rank == 0 and args.cpu_baseline_seconds > 0:
        log(f"timing the oracle on the host ({blas_info()})")
        for n in names:
            wl = WORKLOADS[n]
            layer = oracle_layer(syn, wl["fmt"], wl["bias"], nvq)
            c = cpu_oracle_config(layer, inputs[n],
                                  syn.norm_weight() if args.block else None, prefill=wl["T"] > 64)
            entries[n]["cpu_oracle"] = c
            log(f"oracle {n}: {c['us_per_layer']:.0f} us/layer (all cores), "
                f"{c['us_per_layer_1thread']} us (1 thread)")
        h = entries[headline]["cpu_oracle"]
        cores = len(os.sched_getaffinity(0))
        cpu = {"value": h["us_per_layer"], "unit": "us/layer", "cores": h["blas_threads"],
               "kind": "oracle",
               "sample": f"{WORKLOADS[headline]['T']} tokens of the {headline} workload, "
                         f"{h['form']}; bf16->fp64 weight conversion done once, outside the "
                         f"timed runs; BLAS threads = the {cores} cores of the affinity mask",
               "value_1thread": h["us_per_layer_1thread"],
               "tokens_per_s": h["tokens_per_s"],
               "affinity_cores": cores, "blas": blas_info()}

    e = entries[headline]
    wl = WORKLOADS[headline]
    config = {"workload": e["workload"], "T": wl["T"], "hidden": H, "n_experts": E,
              "top_k": K_TOP, "inter": I, "shared_experts": 1, "router_bias": wl["bias"],
              "seed": args.seed, "n_active": e["n_active"], "layer_copies": args.copies,
              "timing": "one HIP-graph replay of K steps",
              **({"prenorm_block": {"norm": "RMSNorm", "eps": EPS, "residual_add": True}}
                 if args.block else {})}
    result = common_result(
        args, e["us_per_layer"],
        "bf16" if wl["fmt"] == "bf16" else "nvfp4 weights (e2m1 + e4m3 scales), bf16 activations",
        config)
    result.update({k: e[k] for k in ("tokens_per_s", "layer_algorithmic_bytes", "layer_GBps",
                                     "layer_hbm_frac", "layer_algorithmic_flops", "kernels_us",
                                     "eager_wall_us_per_step")})
    result["kernel_timing"] = ("start/stop timestamps of each kernel's execution "
                               "(hipExtLaunchKernelGGL events), averaged over K eager steps")
    if "target" in e:
        result["target"] = e["target"]
    result["roofline"] = e["roofline"]
    if cpu is not None:
        result["cpu_baseline"] = cpu
    if calib is not None:
        result["hbm_calibration"] = calib
    if len(entries) > 1:
        result["per_config"] = entries
    elif "cpu_oracle" in e:
        result["cpu_oracle"] = e["cpu_oracle"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

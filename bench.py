"""Benchmark of the small-batch W4A16 sigmoid-routed MoE decode layer on one
MI355X.

Default workload: one MoE layer (hidden 2048, 256 routed experts of
intermediate 512 plus one shared expert, sigmoid top-6, NVFP4 weights, BF16
activations) decoding one token.  A "step" is one token through a stack of L
copies of the layer (distinct device copies of full 256-expert layers), each
layer computing x + MoE(RMSNorm(x)) on the previous layer's output (the
pre-norm residual block of the model), enqueued by one moe_decode_step call
and replayed as one HIP graph.  The selected-weight footprint of a step
(L x 13.4 MB) is far above the 256 MB Infinity Cache, so the weights stream
from HBM.  Reported value: achieved HBM GB/s on the selected-weight bytes
(router + 6 selected experts + shared expert), with microseconds per layer
beside it; batch-8 figures (Zipf-biased router) are reported alongside.

With the default workload the line also carries "prefill": one NVFP4 MoE
layer over 8192 prompt tokens (Zipf-biased router), timed over whole
moe_prefill_layer calls, with its rate against the BF16 matrix-core peak.

--workload step49: the model's decode step instead: 2 dense SwiGLU layers
(intermediate 5632) and 47 MoE layers, independent seeded weights, RMSNorm
before each, batch 1, one HIP graph.

Prints one JSON line.  Inputs are synthetic and seeded (see synth/).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, K = 2048, 512, 256, 6
NVFP4_MATRIX = I * H * 9 // 16                      # 589,824 B
EXPERT_BYTES = 3 * NVFP4_MATRIX                      # 1,769,472 B
ROUTER_BYTES = E * H * 2 + E * 4                     # BF16 weights + FP32 bias
DENSE_BYTES = 3 * (5632 * H * 9 // 16) + 12          # one dense layer, NVFP4
HBM_PEAK_GBS = 8000.0                                # MI355X HBM3E, published
COUNTERS = os.path.join(ROOT, "profiles", "decode_hbm_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "w4a16_routed_expert_sigmoid_amd", "csrc", f)
                  for f in ("decode.hip", "common.h")]


def selected_bytes(distinct):
    """Algorithmic bytes of one MoE layer call: the router, the distinct
    selected experts and the shared expert (with their FP32 tensor scales)."""
    return ROUTER_BYTES + (distinct + 1) * (EXPERT_BYTES + 12)


def kernel_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per k_layer_b1 launch (batch 1) from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    m = re.search(r"^source_sha:\s*(\w+)", text, re.M)
    t = re.search(r"^k_layer_b1_traffic_bytes:\s*(\d+)", text, re.M)
    if not m or not t or m.group(1) != kernel_source_sha():
        return None
    return int(t.group(1))


def prefill_flops(T, k=K):
    """Algorithmic FLOPs of one prefill call: router GEMM, gate/up and down
    of the T*k routed rows and the T shared rows (2 per multiply-add)."""
    rows = T * k + T
    return 2 * T * E * H + 2 * rows * (2 * I) * H + 2 * rows * H * I


MFMA_BF16_PEAK_TFLOPS = 2500.0                       # MI355X dense BF16, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["layer", "step49"], default="layer")
    p.add_argument("--layers", type=int, default=128, help="layer copies per step (cache hygiene)")
    p.add_argument("--distinct-layers", type=int, default=4, help="independently generated layers")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--prefill-tokens", type=int, default=8192)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill leg")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode layer runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    side = torch.cuda.Stream()  # a non-default stream: graph capture needs one
    with torch.cuda.stream(side):
        out = run(args, dev)
    print(json.dumps(out), flush=True)


def log(m):
    print(f"[bench] {m}", file=sys.stderr, flush=True)


def run(args, dev):
    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    names = ("router_w", "router_b", "w_gate", "w_up", "w_down", "w_scale", "sh_gate", "sh_up", "sh_down",
             "sh_scale", "norm_gain")

    def weights_of(t, bias=None):
        w = moe.moe_layer_weights()
        for n in names:
            v = t.get(n)
            setattr(w, n, None if v is None else v.data_ptr())
        if bias is not None:
            w.router_b = bias.data_ptr()
        return w

    # The prefill leg runs first, before the decode layer copies take tens of
    # GB of device memory.
    pf = None
    if args.workload == "layer" and not args.no_prefill:
        pf = run_prefill(args, dev)
        torch.cuda.empty_cache()

    # ---- layers on the device
    t0 = time.time()
    if args.workload == "layer":
        base = [moe.DeviceLayer(synth.make_layer(j, bias="zero", norm=True), device=dev)
                for j in range(args.distinct_layers)]
        insts = [{n: v.clone() for n, v in base[i % len(base)].t.items()} for i in range(args.layers)]
        descs = [base[0].desc] * args.layers
        del base
    else:
        insts, descs = [], []
        for j in range(49):
            L = (synth.make_layer(j, inter=0, shared_inter=5632, n_experts=0, norm=True) if j < 2
                 else synth.make_layer(j, bias="zero", norm=True))
            d = moe.DeviceLayer(L, device=dev)
            insts.append(d.t)
            descs.append(d.desc)
            del L
    torch.cuda.synchronize()
    nbytes = sum(v.numel() * v.element_size() for t in insts for v in t.values())
    n_layers = len(insts)
    log(f"{n_layers} layers, {nbytes / 1e9:.1f} GB on device, built in {time.time() - t0:.1f}s")
    zipf = torch.from_numpy(synth.zipf_offset(E)).to(dev)

    def run_pool(B, zipf_bias):
        wts = [weights_of(t, zipf if (zipf_bias and descs[i].n_experts) else None) for i, t in enumerate(insts)]
        x = torch.from_numpy(synth.tokens(B, H, stream=1000).view(np.int16)).to(dev)
        y = torch.empty_like(x)
        ws = torch.zeros(moe.moe_decode_step_workspace_bytes(descs, B), dtype=torch.uint8, device=dev)
        g = torch.cuda.CUDAGraph()
        moe.moe_decode_step(descs, wts, x, B, y, ws, ws.numel())
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            moe.moe_decode_step(descs, wts, x, B, y, ws, ws.numel())
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps
        nonfinite = not torch.isfinite(y.view(torch.bfloat16).float()).all().item()

        # Per-layer calls (the same computation), eager, with HIP events
        # attached to each kernel dispatch (start/stop of its execution), and
        # the distinct experts per layer from the top-k outputs.
        acts = [x] + [torch.empty_like(x) for _ in range(n_layers)]
        ws1 = torch.zeros(max(moe.moe_decode_workspace_bytes(d, B) for d in descs), dtype=torch.uint8, device=dev)
        idx = torch.zeros((n_layers, B, K), dtype=torch.int32, device=dev)
        tw = torch.zeros((n_layers, B, K), dtype=torch.float32, device=dev)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_layers)]
        for row in evs:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        st = np.zeros(3)
        nst = 0
        for _ in range(3):
            for i in range(n_layers):
                moe.moe_set_stage_events(evs[i])
                has_k = descs[i].n_experts > 0
                moe.moe_decode_layer(descs[i], wts[i], acts[i], B, 1, acts[i + 1], idx[i] if has_k else None,
                                     tw[i] if has_k else None, ws1, ws1.numel())
            moe.moe_set_stage_events(None)
            torch.cuda.synchronize()
            for i in range(n_layers):
                if descs[i].n_experts == 0:
                    continue
                r = evs[i]
                st += [r[0].elapsed_time(r[1]), r[2].elapsed_time(r[3]), r[4].elapsed_time(r[5])]
                nst += 1
        stage_us = (st / max(nst, 1) * 1e3).tolist()
        same = torch.equal(acts[-1], y)
        moe_layers = [i for i in range(n_layers) if descs[i].n_experts > 0]
        distinct = [len(np.unique(idx[i].cpu().numpy())) for i in moe_layers]
        return dict(ms_step=ms_step, distinct=distinct, stage_us=stage_us, nonfinite=nonfinite,
                    step_equals_layers=bool(same))

    r1 = run_pool(1, False)
    log(f"batch 1: {r1['ms_step'] * 1e3 / n_layers:.2f} us/layer, stages {r1['stage_us']}")
    r8 = None
    if args.workload == "layer":
        r8 = run_pool(8, True)
        log(f"batch 8: {r8['ms_step'] * 1e3 / n_layers:.2f} us/layer, stages {r8['stage_us']}")

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    n_moe = sum(1 for d in descs if d.n_experts > 0)
    n_dense = n_layers - n_moe
    us1 = r1["ms_step"] * 1e3 / n_layers
    step_bytes = sum(selected_bytes(d) for d in r1["distinct"]) + n_dense * DENSE_BYTES
    gbs1 = step_bytes / (r1["ms_step"] * 1e-3) / 1e9

    # batch 1: one kernel per layer (router, gate/up and down of the 6
    # selected experts and the shared expert)
    ex_us = r1["stage_us"][1]
    ex_gbs = selected_bytes(6) / (ex_us * 1e-6) / 1e9
    traffic = measured_traffic()
    roofline = dict(bound="hbm", kernel="k_layer_b1<nvfp4> (router, then gate/up and down of 6 selected + shared "
                    "expert, 1 token)",
                    achieved=round(ex_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ex_gbs / HBM_PEAK_GBS, 4),
                    traffic=traffic, algorithmic_bytes_per_launch=selected_bytes(6), avg_launch_us=round(ex_us, 3))

    cpu = None
    if not args.no_cpu:
        import oracle
        Lh = synth.make_layer(0, wtype="nvfp4", bias="zero")
        n, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and n < 2000:
            xh = synth.tokens(1, H, stream=5000 + n)
            c0 = time.perf_counter()
            oracle.moe_tokens(Lh, xh)
            t_cpu += time.perf_counter() - c0
            n += 1
        us_cpu = t_cpu / n * 1e6
        cpu = dict(value=round(selected_bytes(6) / (us_cpu * 1e-6) / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                   sample=f"{n} batch-1 tokens through one full NVFP4 MoE layer, FP64, single thread",
                   us_per_layer=round(us_cpu, 1))

    if args.workload == "layer":
        workload = ("one NVFP4 MoE decode layer, batch 1 (hidden 2048, 256 experts top-6 + shared, intermediate "
                    "512); step = one token through a chained stack of %d pre-norm layer copies "
                    "(x + MoE(RMSNorm(x))) in one HIP graph" % n_layers)
    else:
        workload = ("decode step of the MoE stack, batch 1: 2 dense SwiGLU (intermediate 5632) + 47 NVFP4 MoE "
                    "layers, RMSNorm before each, independent seeded weights, one HIP graph")
    out = {
        "metric": "MoE-layer decode us + achieved HBM GB/s (selected weights), batch 1 and 8",
        "value": round(gbs1, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "weights": "nvfp4 (E2M1, E4M3 per 16, FP32 per tensor); activations bf16; fp32 accumulation",
                   "layers_per_step": n_layers, "device_weight_gb": round(nbytes / 1e9, 2)},
        "us_per_layer": round(us1, 3),
        "tokens_per_s": round(1e3 / r1["ms_step"], 1) if args.workload == "step49" else round(1e6 / us1, 1),
        "selected_bytes_per_step": int(step_bytes),
        "hbm_frac": round(gbs1 / HBM_PEAK_GBS, 4),
        "stage_us": {"layer_kernel": round(r1["stage_us"][1], 3)},
        "step_equals_layer_calls": r1["step_equals_layers"],
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if r8 is not None:
        us8 = r8["ms_step"] * 1e3 / n_layers
        bytes8 = float(np.mean([selected_bytes(d) for d in r8["distinct"]]))
        gbs8 = bytes8 / (us8 * 1e-6) / 1e9
        out["batch8"] = {"us_per_layer": round(us8, 3), "GBps": round(gbs8, 1),
                         "hbm_frac": round(gbs8 / HBM_PEAK_GBS, 4),
                         "distinct_experts_mean": round(float(np.mean(r8["distinct"])), 2),
                         "tokens_per_s": round(8e6 / us8, 1), "stage_us": [round(v, 3) for v in r8["stage_us"]],
                         "step_equals_layer_calls": r8["step_equals_layers"]}
    if pf is not None:
        out["prefill"] = pf
    if r1["nonfinite"] or (r8 is not None and r8["nonfinite"]) or (pf is not None and pf["nonfinite"]):
        out["warning"] = "non-finite outputs"
    return out


def run_prefill(args, dev):
    """One NVFP4 MoE layer over T prompt tokens (Zipf-biased router), timed
    over whole moe_prefill_layer calls with inputs resident on the device."""
    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    T = args.prefill_tokens
    d = moe.DeviceLayer(synth.make_layer(0, wtype="nvfp4", bias="zipf"), device=dev)
    x = torch.from_numpy(synth.tokens(T, H, stream=2000).view(np.int16)).to(dev)
    y = torch.empty_like(x)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    ws = torch.zeros(moe.moe_prefill_workspace_bytes(d.desc, T), dtype=torch.uint8, device=dev)

    def call():
        moe.moe_prefill_layer(d.desc, d.weights, x, T, 0, y, idx, w, ws, ws.numel())

    # warm up for a quarter second (at least 3 calls): the first tens of
    # milliseconds of a process run at lower clocks
    t_w, n_w = time.time(), 0
    while n_w < 3 or time.time() - t_w < 0.25:
        call()
        torch.cuda.synchronize()
        n_w += 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.prefill_steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.prefill_steps
    flops = prefill_flops(T)
    tflops = flops / (ms * 1e-3) / 1e12
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=E)
    log(f"prefill {T} tokens: {ms:.3f} ms, {tflops:.1f} TFLOP/s")
    return {"tokens": T, "ms_per_layer": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "gflop": round(flops / 1e9, 2), "tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "rows_per_expert_min_mean_max": [int(counts.min()), round(float(counts.mean()), 1), int(counts.max())],
            "nonfinite": not torch.isfinite(y.view(torch.bfloat16).float()).all().item()}


if __name__ == "__main__":
    main()

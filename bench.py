"""Benchmark of the small-batch W4A16 sigmoid-routed MoE decode layer on one
MI355X.

Workload: one MoE layer (hidden 2048, 256 routed experts of intermediate 512
plus one shared expert, sigmoid top-6, NVFP4 weights, BF16 activations)
decoding one token.  A "step" is one token through a stack of L copies of
the layer (distinct device copies of full 256-expert layers), each layer
computing x + MoE(RMSNorm(x)) on the previous layer's output (the pre-norm
residual block of the model), captured in one HIP graph, so the selected-weight footprint of a step (L x 13.4 MB) is far
above the 256 MB Infinity Cache and the weights stream from HBM.  Reported value: achieved HBM GB/s on the
selected-weight bytes (router + 6 selected experts + shared expert), with
the microseconds per layer beside it; batch-8 figures on the Zipf-biased
router are reported alongside.

Prints one JSON line.  Inputs are synthetic and seeded (see synth/).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, K = 2048, 512, 256, 6
NVFP4_MATRIX = I * H * 9 // 16                      # 589,824 B
EXPERT_BYTES = 3 * NVFP4_MATRIX                      # 1,769,472 B
ROUTER_BYTES = E * H * 2 + E * 4                     # BF16 weights + FP32 bias
HBM_PEAK_GBS = 8000.0                                # MI355X HBM3E, published


def selected_bytes(distinct):
    """Algorithmic bytes of one layer call: the router, the distinct selected
    experts and the shared expert (with their FP32 tensor scales)."""
    return ROUTER_BYTES + (distinct + 1) * (EXPERT_BYTES + 12)


def gateup_bytes(distinct):
    return (distinct + 1) * (2 * NVFP4_MATRIX + 8)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=128, help="layer copies per step (cache hygiene)")
    p.add_argument("--distinct-layers", type=int, default=4, help="independently generated layers")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode layer runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    side = torch.cuda.Stream()  # a non-default stream: graph capture needs one
    with torch.cuda.stream(side):
        _run(args, np, torch, synth, moe, dev)


def _run(args, np, torch, synth, moe, dev):
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)  # noqa: E731

    # ---- weights: a few generated layers, copied to L device instances
    t0 = time.time()
    base = []
    for j in range(args.distinct_layers):
        L = synth.make_layer(j, wtype="nvfp4", bias="zero", norm=True)
        base.append(moe.DeviceLayer(L, device=dev))
        del L
    zipf = torch.from_numpy(synth.zipf_offset(E)).to(dev)
    log(f"generated {args.distinct_layers} layers in {time.time() - t0:.1f}s")
    names = ("router_w", "w_gate", "w_up", "w_down", "w_scale", "sh_gate", "sh_up", "sh_down", "sh_scale",
             "norm_gain")
    inst = []
    for i in range(args.layers):
        src = base[i % len(base)]
        t = {n: src.t[n].clone() for n in names}
        t["router_b"] = src.t["router_b"].clone()
        inst.append(t)
    torch.cuda.synchronize()
    nbytes = sum(v.numel() * v.element_size() for t in inst for v in t.values())
    log(f"{args.layers} layer instances, {nbytes / 1e9:.1f} GB on device")

    def weights_of(t, bias):
        w = moe.moe_layer_weights()
        for n in names:
            setattr(w, n, t[n].data_ptr())
        w.router_b = bias.data_ptr()
        return w

    desc = base[0].desc

    def run_pool(B, zipf_bias):
        # act[i] -> layer i -> act[i + 1]: a chained stack with residual adds
        act = [torch.from_numpy(synth.tokens(B, H, stream=1000).view(np.int16)).to(dev)]
        act += [torch.empty_like(act[0]) for _ in range(args.layers)]
        xs, ys = act[:-1], act[1:]
        idx = torch.empty((args.layers, B, K), dtype=torch.int32, device=dev)
        tw = torch.empty((args.layers, B, K), dtype=torch.float32, device=dev)
        ws = torch.zeros(moe.moe_decode_workspace_bytes(desc, B), dtype=torch.uint8, device=dev)
        ws_ = [weights_of(t, zipf if zipf_bias else t["router_b"]) for t in inst]

        def step(events=None):
            for i in range(args.layers):
                if events is not None:
                    moe.moe_set_stage_events(events[i])
                moe.moe_decode_layer(desc, ws_[i], xs[i], B, 1, ys[i], idx[i], tw[i], ws, ws.numel())
            if events is not None:
                moe.moe_set_stage_events(None)

        step()
        torch.cuda.synchronize()
        distinct = [len(np.unique(idx[i].cpu().numpy())) for i in range(args.layers)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_step = e0.elapsed_time(e1) / args.steps

        # Per-stage kernel durations: HIP events around each stage, enqueued
        # behind a sleeping kernel so the queue is full and launches are
        # back to back on the GPU, averaged over all instances and rounds.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.layers)]
        for row in evs:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        st = np.zeros(3)
        rounds = 3
        for _ in range(rounds):
            torch.cuda._sleep(50_000_000)
            step(evs)
            torch.cuda.synchronize()
            for row in evs:
                st += [row[0].elapsed_time(row[1]), row[2].elapsed_time(row[3]), row[4].elapsed_time(row[5])]
        st_us = st / (rounds * args.layers) * 1e3
        ybad = not torch.isfinite(ys[-1].view(torch.bfloat16).float()).all().item()
        return dict(ms_step=ms_step, wall=wall, distinct=distinct, stage_us=st_us.tolist(), nonfinite=ybad)

    r1 = run_pool(1, False)
    log(f"batch 1: {r1['ms_step'] * 1e3 / args.layers:.2f} us/layer, stages {r1['stage_us']}")
    r8 = run_pool(8, True)
    log(f"batch 8: {r8['ms_step'] * 1e3 / args.layers:.2f} us/layer, stages {r8['stage_us']}")

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    us1 = r1["ms_step"] * 1e3 / args.layers
    bytes1 = np.mean([selected_bytes(d) for d in r1["distinct"]])
    gbs1 = bytes1 / (us1 * 1e-6) / 1e9
    us8 = r8["ms_step"] * 1e3 / args.layers
    d8 = float(np.mean(r8["distinct"]))
    bytes8 = np.mean([selected_bytes(d) for d in r8["distinct"]])
    gbs8 = bytes8 / (us8 * 1e-6) / 1e9

    # roofline of the dominant kernel (gate/up: 8.26 MB of the 13.4 MB)
    gu_us = r1["stage_us"][1]
    gu_gbs = gateup_bytes(6) / (gu_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", kernel="k_gateup (gate+up GEMV, SiLU*up)", achieved=round(gu_gbs, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gu_gbs / HBM_PEAK_GBS, 4),
                    traffic=None, algorithmic_bytes_per_launch=gateup_bytes(6), avg_launch_us=round(gu_us, 3))

    cpu = None
    if not args.no_cpu:
        import oracle
        Lh = synth.make_layer(0, wtype="nvfp4", bias="zero")
        n, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and n < 2000:
            x = synth.tokens(1, H, stream=5000 + n)
            c0 = time.perf_counter()
            oracle.moe_tokens(Lh, x)
            t_cpu += time.perf_counter() - c0
            n += 1
        us_cpu = t_cpu / n * 1e6
        cpu = dict(value=round(selected_bytes(6) / (us_cpu * 1e-6) / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                   sample=f"{n} batch-1 tokens through one full NVFP4 layer, FP64, single thread",
                   us_per_layer=round(us_cpu, 1))

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
        "config": {
            "workload": "one NVFP4 MoE decode layer, batch 1 (hidden 2048, 256 experts top-6 + shared, "
                        "intermediate 512); step = one token through a chained stack of %d pre-norm layer "
                        "copies (x + MoE(RMSNorm(x))) in one HIP graph" % args.layers,
            "weights": "nvfp4 (E2M1, E4M3 per 16, FP32 per tensor); activations bf16; fp32 accumulation",
            "layers_per_step": args.layers,
            "device_weight_gb": round(nbytes / 1e9, 2),
        },
        "us_per_layer": round(us1, 3),
        "tokens_per_s": round(1e6 / us1, 1),
        "selected_bytes_per_layer": int(bytes1),
        "hbm_frac": round(gbs1 / HBM_PEAK_GBS, 4),
        "stage_us": {"router_topk": round(r1["stage_us"][0], 3), "gateup": round(r1["stage_us"][1], 3),
                     "down_combine": round(r1["stage_us"][2], 3)},
        "batch8": {"us_per_layer": round(us8, 3), "GBps": round(gbs8, 1), "hbm_frac": round(gbs8 / HBM_PEAK_GBS, 4),
                   "distinct_experts_mean": round(d8, 2), "tokens_per_s": round(8e6 / us8, 1),
                   "stage_us": [round(v, 3) for v in r8["stage_us"]]},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if r1["nonfinite"] or r8["nonfinite"]:
        out["warning"] = "non-finite outputs"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the small-batch W4A16 sigmoid-routed MoE decode layer on one
MI355X.

Default workload (the headline value): one NVFP4 MoE layer (hidden 2048,
256 routed experts of intermediate 512 plus one shared expert, sigmoid
top-6, BF16 activations) decoding one token.  A "step" is one token through
a stack of L device copies of full 256-expert layers, each computing
x + MoE(RMSNorm(x)) on the previous layer's output (the pre-norm residual
block of the model), enqueued by one moe_decode_step call and replayed as
one HIP graph.  The selected-weight footprint of a step (L x 13.4 MB) is far
above the 256 MB Infinity Cache, so the weights stream from HBM.  Value:
achieved HBM GB/s on the selected-weight bytes (router + 6 selected experts
+ shared expert), with microseconds per layer beside it.

The same line carries every configuration the layer is measured on, under
"configs": BF16 weights at batch 1, NVFP4 at batch 1, NVFP4 at batch 8 with
a Zipf-biased router, the model's decode step (2 dense SwiGLU layers of
intermediate 5632 and 47 MoE layers, one HIP graph), and the 8192-token
prefill of one layer on the matrix cores.  Also: the measured HBM read
ceiling (a streaming-read kernel), the roofline of the batch-1 layer kernel
and the CPU oracle's time on the host cores.

Beside the MoE layer: the dense NVFP4 projection (LM-head and fused-QKV
shapes) and the decode attention of one 49-layer step at 100K context (14
full-context layers, 35 sliding-window layers; Q/K norm, RoPE and KV write,
then attention with sinks), at batch 1 and 8.

--workload step49: the model's decode step alone, with 47 independently
generated MoE layers instead of device copies of a few.
--attn-only: the attention leg alone (for profiling).

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
EXPERT_BYTES_BF16 = 3 * I * H * 2                    # 6,291,456 B
ROUTER_BYTES = E * H * 2 + E * 4                     # BF16 weights + FP32 bias
DENSE_BYTES = 3 * (5632 * H * 9 // 16) + 12          # one dense layer, NVFP4
HBM_PEAK_GBS = 8000.0                                # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0                       # MI355X dense BF16, published
COUNTERS = os.path.join(ROOT, "profiles", "decode_hbm_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "w4a16_routed_expert_sigmoid_amd", "csrc", f)
                  for f in ("decode.hip", "mm_rows.h", "common.h", "shapes.h")]


def selected_bytes(distinct, expert_bytes=EXPERT_BYTES, scales=12):
    """Algorithmic bytes of one MoE layer call: the router, the distinct
    selected experts and the shared expert (with their FP32 tensor scales)."""
    return ROUTER_BYTES + (distinct + 1) * (expert_bytes + scales)


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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["layer", "step49"], default="layer")
    p.add_argument("--layers", type=int, default=128, help="NVFP4 layer copies per step (cache hygiene)")
    p.add_argument("--bf16-layers", type=int, default=24, help="BF16 layer copies per step (cache hygiene)")
    p.add_argument("--distinct-layers", type=int, default=4, help="independently generated MoE layers")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="wall time of each oracle leg")
    p.add_argument("--prefill-tokens", type=int, default=8192)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill leg")
    p.add_argument("--no-bf16", action="store_true", help="skip the BF16-weight leg")
    p.add_argument("--no-gemv", action="store_true", help="skip the dense-projection leg")
    p.add_argument("--no-mid", action="store_true", help="skip the 16..256-token leg")
    p.add_argument("--no-attn", action="store_true", help="skip the decode-attention leg")
    p.add_argument("--attn-ctx", type=int, default=100000,
                   help="decode position of the attention leg (the pages' 100K context)")
    p.add_argument("--attn-batches", default="1,8", help="batches of the attention leg")
    p.add_argument("--attn-only", action="store_true",
                   help="run only the decode-attention leg and print its results (profiling)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a 1 GiB streaming read and a 1 GiB copy (counter calibration under rocprofv3 --pmc)")
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
        if args.attn_only:
            out = {"attn_step_100k": run_attention(args, dev)}
            if args.copy_probe:
                copy_probe(dev)
        else:
            out = run(args, dev)
    print(json.dumps(out), flush=True)


def log(m):
    print(f"[bench] {m}", file=sys.stderr, flush=True)


def weights_of(moe, t, bias=None):
    w = moe.moe_layer_weights()
    for n, _ in moe.moe_layer_weights._fields_:
        v = t.get(n)
        setattr(w, n, None if v is None else v.data_ptr())
    if bias is not None:
        w.router_b = bias.data_ptr()
    return w


def time_stack(args, dev, insts, descs, B, bias, label):
    """One token batch through the stack as one HIP graph (timed over
    args.steps replays), then the same layers as eager calls with events on
    their kernel dispatches.  Returns timings, distinct experts per MoE
    layer and the wait status of both workspaces."""
    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    n_layers = len(insts)
    wts = [weights_of(moe, t, bias if (bias is not None and descs[i].n_experts) else None)
           for i, t in enumerate(insts)]
    x = torch.from_numpy(synth.tokens(B, H, stream=1000).view(np.int16)).to(dev)
    y = torch.empty_like(x)
    ws = torch.zeros(moe.moe_decode_step_workspace_bytes(descs, B), dtype=torch.uint8, device=dev)
    status = torch.full((2,), -1, dtype=torch.int32, device=dev)
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
    moe.moe_decode_wait_status(ws, status[0:1])
    nonfinite = not torch.isfinite(y.view(torch.bfloat16).float()).all().item()

    # One token: the same stack through the persistent step (runs of MoE
    # layers in one kernel each), its own graph, timed the same way.
    ms_persist, persist_same, persist_wait = None, None, 0
    if B == 1:
        wsp = torch.zeros(moe.moe_decode_step_persistent_workspace_bytes(descs, B), dtype=torch.uint8, device=dev)
        yp = torch.empty_like(x)
        moe.moe_decode_step_persistent(descs, wts, x, B, yp, wsp, wsp.numel())
        torch.cuda.synchronize()
        gp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp):
            moe.moe_decode_step_persistent(descs, wts, x, B, yp, wsp, wsp.numel())
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            gp.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            gp.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_persist = e0.elapsed_time(e1) / args.steps
        persist_same = bool(torch.equal(yp, y))
        st_p = torch.full((1,), -1, dtype=torch.int32, device=dev)
        moe.moe_decode_wait_status(wsp, st_p)
        persist_wait = int(st_p.item())
        del wsp, gp

    # Per-layer calls (the same computation), eager, with HIP events
    # attached to each kernel dispatch (start/stop of its execution), and
    # the distinct experts per layer from the top-k outputs.
    acts = [x] + [torch.empty_like(x) for _ in range(n_layers)]
    ws1 = torch.zeros(max(moe.moe_decode_workspace_bytes(d, B) for d in descs), dtype=torch.uint8, device=dev)
    idx = torch.zeros((n_layers, B, K), dtype=torch.int32, device=dev)
    tw = torch.zeros((n_layers, B, K), dtype=torch.float32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_layers)]
    st_any = torch.zeros(1, dtype=torch.int32, device=dev)
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    st = np.zeros(3)
    nst = 0
    for _ in range(3):
        for i in range(n_layers):
            has_k = descs[i].n_experts > 0
            moe.moe_decode_layer_timed(descs[i], wts[i], acts[i], B, 1, acts[i + 1], idx[i] if has_k else None,
                                       tw[i] if has_k else None, ws1, ws1.numel(), evs[i])
            moe.moe_decode_wait_status(ws1, status[1:2])
            st_any.bitwise_or_(status[1:2])
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
    wait = int(status[0].item()) | int(st_any.item()) | persist_wait
    log(f"{label}: {ms_step * 1e3 / n_layers:.2f} us/layer in the graph, stage kernels {stage_us} us, "
        f"wait status {wait}" + (f"; persistent step {ms_persist * 1e3 / n_layers:.2f} us/layer, "
                                 f"equal {persist_same}" if ms_persist else ""))
    return dict(ms_step=ms_step, distinct=distinct, stage_us=stage_us, nonfinite=nonfinite,
                step_equals_layers=bool(same), wait_status=wait, ms_persist=ms_persist, persist_same=persist_same)


def stream_ceiling(dev):
    """Best read bandwidth of the streaming-read probe over a 4 GiB buffer
    (1024 to 8192 blocks of 256 threads)."""
    import torch

    import w4a16_routed_expert_sigmoid_amd as moe

    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        for _ in range(2):
            moe.moe_probe_hbm_read(buf, n, blocks, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            moe.moe_probe_hbm_read(buf, n, blocks, sink)
        e1.record()
        torch.cuda.synchronize()
        gbs = n / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, blocks)
    del buf
    log(f"stream read ceiling {best[0]:.0f} GB/s ({best[1]} blocks)")
    return {"GBps": round(best[0], 1), "bytes": n, "blocks": best[1], "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4),
            "kernel": "k_probe_read (moe_probe_hbm_read): 16-byte nontemporal loads, grid-stride, 4 in flight"}


def copy_probe(dev):
    """Known sizes for scaling the traffic counters: a 1 GiB streaming read,
    then a 1 GiB device copy (1 GiB read + 1 GiB written)."""
    import torch

    import w4a16_routed_expert_sigmoid_amd as moe
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_probe_hbm_read(a, a.numel(), 2048, sink)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def cpu_baseline(seconds):
    """The oracle (FP64, plain C) on one host thread and on every host thread
    (one owner per token, so both give the same bits), each for about
    `seconds` of wall time on whole batch-1 tokens through one full NVFP4
    MoE layer."""
    import oracle
    import synth

    Lh = synth.make_layer(0, wtype="nvfp4", bias="zero")

    def leg(threads):
        n, t, s = 0, 0.0, 0
        while t < seconds and n < 200000:
            m = max(threads, 1) * (1 if threads == 1 else 4)
            xh = synth.tokens(m, H, stream=5000 + s)
            c0 = time.perf_counter()
            oracle.moe_tokens(Lh, xh, threads=threads)
            t += time.perf_counter() - c0
            n += m
            s += 1
        return n, t

    n1, t1 = leg(1)
    nt = oracle.host_threads()
    nn, tn = leg(nt)
    us1, usn = t1 / n1 * 1e6, tn / nn * 1e6
    gb = selected_bytes(6)
    log(f"oracle: {us1:.0f} us/token on 1 thread, {usn:.0f} us/token on {nt} threads")
    return dict(value=round(gb / (usn * 1e-6) / 1e9, 4), unit="GB/s", cores=nt, kind="oracle",
                sample=f"{nn} batch-1 tokens through one full NVFP4 MoE layer (FP64) on {nt} host threads, "
                       f"{tn:.1f} s wall",
                us_per_token=round(usn, 1),
                single_thread={"value": round(gb / (us1 * 1e-6) / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "us_per_token": round(us1, 1), "sample": f"{n1} tokens, {t1:.1f} s"})


def clone_pool(base, n):
    return [{k: v.clone() for k, v in base[i % len(base)].t.items()} for i in range(n)]


def run(args, dev):
    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    configs = {}
    # The prefill leg runs first, before the decode layer copies take tens of
    # GB of device memory.
    pf = None
    if args.workload == "layer" and not args.no_prefill:
        pf = run_prefill(args, dev)
        configs["prefill_8192_nvfp4"] = pf
        torch.cuda.empty_cache()

    if args.workload == "layer" and not args.no_gemv:
        configs["dense_gemv_nvfp4"] = run_gemv(args, dev)
        torch.cuda.empty_cache()

    if args.workload == "layer" and not args.no_attn:
        configs["attn_step_100k"] = run_attention(args, dev)
        torch.cuda.empty_cache()

    zipf = torch.from_numpy(synth.zipf_offset(E)).to(dev)
    t0 = time.time()
    dense = [moe.DeviceLayer(synth.make_layer(j, inter=0, shared_inter=5632, n_experts=0, norm=True), device=dev)
             for j in range(2)]
    if args.workload == "layer":
        base = [moe.DeviceLayer(synth.make_layer(2 + j, bias="zero", norm=True), device=dev)
                for j in range(args.distinct_layers)]
        pool = clone_pool(base, args.layers)
        mdesc = base[0].desc
        del base
    else:
        pool, mdesc = [], None
        for j in range(47):
            d = moe.DeviceLayer(synth.make_layer(2 + j, bias="zero", norm=True), device=dev)
            pool.append(d.t)
            mdesc = d.desc
    torch.cuda.synchronize()
    nbytes = sum(v.numel() * v.element_size() for t in pool for v in t.values())
    log(f"{len(pool)} NVFP4 MoE layers, {nbytes / 1e9:.1f} GB on device, built in {time.time() - t0:.1f}s")

    def gb_per_s(distinct, ms, expert_bytes, scales, extra):
        b = sum(selected_bytes(d, expert_bytes, scales) for d in distinct) + extra
        return b, b / (ms * 1e-3) / 1e9

    ceiling = stream_ceiling(dev)
    ceil_gbs = ceiling["GBps"]
    for v in configs.get("attn_step_100k", {}).values():
        v["full_decode_stream_frac"] = round(v["full_decode_GBps"] / ceil_gbs, 4)

    def summary(r, n_layers, B, expert_bytes=EXPERT_BYTES, scales=12, extra=0):
        b, gbs = gb_per_s(r["distinct"], r["ms_step"], expert_bytes, scales, extra)
        us = r["ms_step"] * 1e3 / n_layers
        return {"us_per_layer": round(us, 3), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "stream_frac": round(gbs / ceil_gbs, 4), "tokens_per_s": round(B * 1e6 / us, 1),
                "layers_per_step": n_layers, "ms_per_step": round(r["ms_step"], 4),
                "selected_bytes_per_step": int(b),
                "distinct_experts_mean": round(float(np.mean(r["distinct"])), 2) if r["distinct"] else None,
                "stage_kernel_us": [round(v, 3) for v in r["stage_us"]],
                "step_equals_layer_calls": r["step_equals_layers"], "wait_status": r["wait_status"],
                "persistent_step_us_per_layer": (round(r["ms_persist"] * 1e3 / n_layers, 3)
                                                 if r["ms_persist"] else None),
                "persistent_step_equals_step": r["persist_same"]}

    warn = []
    if pf is not None and pf["nonfinite"]:
        warn.append("non-finite outputs")
    r1 = None
    if args.workload == "layer":
        descs = [mdesc] * len(pool)
        r1 = time_stack(args, dev, pool, descs, 1, None, "NVFP4 batch 1")
        configs["nvfp4_b1"] = summary(r1, len(pool), 1)
        r8 = time_stack(args, dev, pool, descs, 8, zipf, "NVFP4 batch 8 (Zipf)")
        configs["nvfp4_b8_zipf"] = summary(r8, len(pool), 8)
        # 16 tokens through the same decode kernels (the mid-batch leg below
        # runs 16 tokens through the prefill entry)
        r16 = time_stack(args, dev, pool, descs, 16, zipf, "NVFP4 batch 16 (Zipf)")
        configs["nvfp4_b16_zipf"] = summary(r16, len(pool), 16)
        for r in (r1, r8, r16):
            if r["nonfinite"]:
                warn.append("non-finite outputs")
    if args.workload == "layer" and not args.no_mid:
        configs["mid_batch_nvfp4_zipf"] = run_mid_batch(args, dev, pool, mdesc, zipf, ceil_gbs)
    # the model's decode step: 2 dense layers, then 47 MoE layers
    step_pool = [d.t for d in dense] + [pool[i % len(pool)] for i in range(47)]
    step_descs = [d.desc for d in dense] + [mdesc] * 47
    r49 = time_stack(args, dev, step_pool, step_descs, 1, None, "49-layer step batch 1")
    s49 = summary(r49, 49, 1, extra=2 * DENSE_BYTES + 49 * H * 2)   # + the 49 RMSNorm gains
    s49["tokens_per_s"] = round(1e3 / r49["ms_step"], 1)
    s49["moe_layers_from"] = ("device copies of %d independently generated layers" % args.distinct_layers
                              if args.workload == "layer" else "47 independently generated layers")
    configs["step49_b1"] = s49
    if r49["nonfinite"]:
        warn.append("non-finite outputs")
    if any(r is not None and r["persist_same"] is False for r in (r1, r49)):
        warn.append("the persistent step's output differs from the step's")
    r1 = r1 if r1 is not None else r49
    del pool, step_pool
    torch.cuda.empty_cache()

    if args.workload == "layer" and not args.no_bf16:
        t0 = time.time()
        bbase = [moe.DeviceLayer(synth.make_layer(2 + j, wtype="bf16", bias="zero", norm=True), device=dev)
                 for j in range(2)]
        bpool = clone_pool(bbase, args.bf16_layers)
        bdesc = bbase[0].desc
        del bbase
        torch.cuda.synchronize()
        log(f"{len(bpool)} BF16 MoE layers built in {time.time() - t0:.1f}s")
        rb = time_stack(args, dev, bpool, [bdesc] * len(bpool), 1, None, "BF16 batch 1")
        configs["bf16_b1"] = summary(rb, len(bpool), 1, expert_bytes=EXPERT_BYTES_BF16, scales=0)
        if rb["nonfinite"]:
            warn.append("non-finite outputs")
        del bpool
        torch.cuda.empty_cache()

    if args.copy_probe:
        copy_probe(dev)

    # batch 1: one kernel per layer (router, gate/up and down of the 6
    # selected experts and the shared expert)
    ex_us = r1["stage_us"][1]
    ex_gbs = selected_bytes(6) / (ex_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", kernel="k_layer_b1<nvfp4> (router, then gate/up and down of 6 selected + shared "
                    "expert, 1 token)",
                    achieved=round(ex_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ex_gbs / HBM_PEAK_GBS, 4),
                    traffic=measured_traffic(), algorithmic_bytes_per_launch=selected_bytes(6),
                    avg_launch_us=round(ex_us, 3), stream_ceiling_GBps=ceil_gbs,
                    frac_of_stream_ceiling=round(ex_gbs / ceil_gbs, 4))

    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)

    head = configs["nvfp4_b1"] if args.workload == "layer" else configs["step49_b1"]
    if args.workload == "layer":
        workload = ("one NVFP4 MoE decode layer, batch 1 (hidden 2048, 256 experts top-6 + shared, intermediate "
                    "512); step = one token through a chained stack of %d pre-norm layer copies "
                    "(x + MoE(RMSNorm(x))) in one HIP graph" % args.layers)
    else:
        workload = ("decode step of the MoE stack, batch 1: 2 dense SwiGLU (intermediate 5632) + 47 NVFP4 MoE "
                    "layers, RMSNorm before each, independent seeded weights, one HIP graph")
    if any(v.get("status") for v in configs.get("attn_step_100k", {}).values()):
        warn.append("attention status non-zero: outputs invalid")
    if any(v.get("fused_equals_prep_decode") is False for v in configs.get("attn_step_100k", {}).values()):
        warn.append("the fused attention layer differs from prep + decode")
    if any(v.get("nonfinite") for k in ("dense_gemv_nvfp4", "mid_batch_nvfp4_zipf", "attn_step_100k")
           for v in configs.get(k, {}).values()):
        warn.append("non-finite outputs")
    gbs1 = head["GBps"]
    wait = max(c.get("wait_status", 0) for c in configs.values() if isinstance(c, dict))
    if wait:
        warn.append(f"a bounded wait gave up (status {wait}): outputs invalid")
    out = {
        "metric": "MoE-layer decode us + achieved HBM GB/s (selected weights), batch 1 and 8",
        "value": gbs1,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "weights": "nvfp4 (E2M1, E4M3 per 16, FP32 per tensor); activations bf16; fp32 accumulation",
                   "layers_per_step": head["layers_per_step"]},
        "us_per_layer": head["us_per_layer"],
        "tokens_per_s": head["tokens_per_s"],
        "hbm_frac": head["hbm_frac"],
        "stream_frac": head["stream_frac"],
        "wait_status": wait,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stream_ceiling": ceiling,
        "configs": configs,
    }
    if warn:
        out["warning"] = "; ".join(sorted(set(warn)))
    return out


def run_mid_batch(args, dev, pool, desc, zipf, ceil_gbs):
    """Batches between the decode path and the long prefill: T tokens
    through moe_prefill_layer on the full NVFP4 layer with the Zipf-biased
    router, one call per layer copy, replayed as one HIP graph over enough
    copies that the selected weights stream from HBM."""
    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    out = {}
    for T in (16, 32, 64, 128, 256):
        x = torch.from_numpy(synth.tokens(T, H, stream=3000 + T).view(np.int16)).to(dev)
        y = torch.empty_like(x)
        idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
        ws = torch.zeros(moe.moe_prefill_workspace_bytes(desc, T), dtype=torch.uint8, device=dev)
        wts = [weights_of(moe, t, zipf) for t in pool]
        moe.moe_prefill_layer(desc, wts[0], x, T, 0, y, idx, w, ws, ws.numel())
        torch.cuda.synchronize()
        distinct = len(np.unique(idx.cpu().numpy()))
        per_call = selected_bytes(distinct)
        n = int(min(len(wts), max(8, -(-(2 << 30) // per_call))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                moe.moe_prefill_layer(desc, wts[i], x, T, 0, y, idx, w, ws, ws.numel())
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n)
        gbs = per_call / (us * 1e-6) / 1e9
        out[f"T{T}"] = {"us_per_layer": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
                        "distinct_experts": distinct, "selected_bytes": int(per_call), "GBps": round(gbs, 1),
                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "stream_frac": round(gbs / ceil_gbs, 4),
                        "tflops": round(prefill_flops(T) / (us * 1e-6) / 1e12, 1), "layer_calls_per_replay": n,
                        "nonfinite": not torch.isfinite(y.view(torch.bfloat16).float()).all().item()}
        log(f"mid batch T={T}: {us:.1f} us/layer, {distinct} distinct experts, {gbs:.0f} GB/s")
        del ws, g
    return out


def run_gemv(args, dev):
    """The dense NVFP4 projection at batch 1 and 8 on an LM-head-sized
    (131072 x 2048) and a fused-QKV-sized (5120 x 2048: 32 query and 4 + 4
    KV heads of 128) matrix: device
    copies of one repacked matrix, rotated so that one graph replay streams
    more than 1 GB of weights from HBM; GB/s on the weight bytes."""
    import numpy as np
    import torch

    import synth
    import w4a16_routed_expert_sigmoid_amd as moe

    out = {}
    for name, rows in (("lm_head_131072x2048", 131072), ("qkv_5120x2048", 5120)):
        cols = H
        m, sc = synth.nvfp4_stack(4242, 0, 1, 1, rows, cols)
        src = torch.from_numpy(m.reshape(-1)).to(dev)
        w0 = torch.empty_like(src)
        moe.moe_repack_nvfp4(src, w0, rows, cols, 1)
        del src
        nbytes = w0.numel()
        copies = max(2, -(-(1 << 30) // nbytes))
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        s = torch.tensor([float(sc[0])], dtype=torch.float32, device=dev)
        for B in (1, 8):
            x = torch.from_numpy(synth.tokens(B, cols, stream=77).view(np.int16)).to(dev)
            y = torch.empty((B, rows), dtype=torch.int16, device=dev)
            g = torch.cuda.CUDAGraph()
            moe.moe_gemv_nvfp4(ws[0], s, rows, cols, x, B, y)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for w in ws:
                    moe.moe_gemv_nvfp4(w, s, rows, cols, x, B, y)
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            reps = 5
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(ws))
            gbs = nbytes / (us * 1e-6) / 1e9
            out[f"{name}_b{B}"] = {"us": round(us, 3), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "weight_bytes": int(nbytes), "copies_per_replay": len(ws),
                                   "nonfinite": not torch.isfinite(y.view(torch.bfloat16).float()).all().item()}
            log(f"gemv {name} B={B}: {us:.2f} us, {gbs:.0f} GB/s")
        del ws, w0
        torch.cuda.empty_cache()
    return out


ATTN_NQ, ATTN_NKV, ATTN_D, ATTN_WINDOW, ATTN_RING = 32, 4, 128, 513, 544


def run_attention(args, dev):
    """Decode attention of one 49-layer step at the pages' decode setting
    (context 100K): 14 full-context layers (no RoPE) attending every
    position and 35 sliding-window layers (513 positions, RoPE, a 544-slot
    ring), GQA 32/4 of 128, sinks, each layer = moe_attn_prep (Q/K norm,
    RoPE, KV write) then moe_attn_decode, all 49 in one HIP graph.  Caches
    hold seeded random BF16 (the full layers' 14 x 205 MB per token stream
    from HBM every step).  Also the full-context decode alone, timed per
    call with events: GB/s on the K and V bytes it must read."""
    import torch

    import w4a16_routed_expert_sigmoid_amd as moe

    ctx = args.attn_ctx                       # position of the decoded token
    span = ctx + 1
    full_slots = -(-span // 32) * 32
    full = moe.moe_attn_desc(ATTN_NQ, ATTN_NKV, ATTN_D, 0, 0, full_slots, 0.0, 1e-6)
    swa = moe.moe_attn_desc(ATTN_NQ, ATTN_NKV, ATTN_D, ATTN_WINDOW, 1, ATTN_RING, 10000.0, 1e-6)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4711)
    out = {}
    for B in [int(b) for b in args.attn_batches.split(",") if b]:
        t0 = time.time()
        layers = []
        for i in range(49):
            is_full = i % 7 >= 5                   # 14 of 49
            d = full if is_full else swa
            slots = full_slots if is_full else ATTN_RING
            n = B * ATTN_NKV * slots * ATTN_D
            L = dict(desc=d, full=is_full, max_ctx=span if is_full else 0,
                     kc=torch.randn(n, device=dev, dtype=torch.bfloat16, generator=gen).view(torch.int16),
                     vc=torch.randn(n, device=dev, dtype=torch.bfloat16, generator=gen).view(torch.int16),
                     qkv=torch.randn(B * (ATTN_NQ + 2 * ATTN_NKV) * ATTN_D, device=dev, dtype=torch.bfloat16,
                                     generator=gen).view(torch.int16),
                     qg=(1 + 0.02 * torch.randn(ATTN_D, device=dev, generator=gen)).bfloat16().view(torch.int16),
                     kg=(1 + 0.02 * torch.randn(ATTN_D, device=dev, generator=gen)).bfloat16().view(torch.int16),
                     sinks=torch.randn(ATTN_NQ, device=dev, generator=gen),
                     q=torch.empty(B * ATTN_NQ * ATTN_D, dtype=torch.int16, device=dev),
                     o=torch.empty(B * ATTN_NQ * ATTN_D, dtype=torch.int16, device=dev))
            L["ws_bytes"] = moe.moe_attn_workspace_bytes(d, B, L["max_ctx"])
            L["ws"] = torch.empty(L["ws_bytes"], dtype=torch.uint8, device=dev)
            layers.append(L)
        pos = torch.full((B,), ctx, dtype=torch.int64, device=dev)
        torch.cuda.synchronize()
        cache_bytes = sum(2 * L["kc"].numel() * 2 for L in layers)
        log(f"attention B={B}: 49 layers, caches {cache_bytes / 1e9:.2f} GB, built in {time.time() - t0:.1f}s")

        def layer_call(L):
            moe.moe_attn_prep(L["desc"], L["qkv"], pos, B, L["qg"], L["kg"], L["q"], L["kc"], L["vc"])
            moe.moe_attn_decode(L["desc"], L["q"], L["kc"], L["vc"], pos, B, L["o"], L["ws"], L["ws_bytes"],
                                max_ctx=L["max_ctx"], sinks=L["sinks"])

        for L in layers:
            layer_call(L)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for L in layers:
                layer_call(L)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps // 5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        step_us = e0.elapsed_time(e1) * 1e3 / reps
        outs = [L["o"].clone() for L in layers]
        # the same step with each layer in one fused call (moe_attn_layer)
        for L in layers:
            moe.moe_attn_layer(L["desc"], L["qkv"], pos, B, L["qg"], L["kg"], L["kc"], L["vc"], L["o"], L["ws"],
                               L["ws_bytes"], max_ctx=L["max_ctx"], sinks=L["sinks"])
        torch.cuda.synchronize()
        fused_same = all(torch.equal(L["o"], o) for L, o in zip(layers, outs))
        gf = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gf):
            for L in layers:
                moe.moe_attn_layer(L["desc"], L["qkv"], pos, B, L["qg"], L["kg"], L["kc"], L["vc"], L["o"],
                                   L["ws"], L["ws_bytes"], max_ctx=L["max_ctx"], sinks=L["sinks"])
        for _ in range(3):
            gf.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            gf.replay()
        e1.record()
        torch.cuda.synchronize()
        fused_us = e0.elapsed_time(e1) * 1e3 / reps
        del gf
        # the full-context decode alone (split + combine kernels), per call
        fulls = [L for L in layers if L["full"]]
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3 * 14)]
        k = 0
        for _ in range(3):
            for L in fulls:
                ev[k][0].record()
                moe.moe_attn_decode(L["desc"], L["q"], L["kc"], L["vc"], pos, B, L["o"], L["ws"], L["ws_bytes"],
                                    max_ctx=L["max_ctx"], sinks=L["sinks"])
                ev[k][1].record()
                k += 1
        torch.cuda.synchronize()
        times = sorted(a.elapsed_time(b) * 1e3 for a, b in ev[14:])   # skip the first pass
        full_us = times[len(times) // 2]
        kv_bytes = B * ATTN_NKV * span * ATTN_D * 2 * 2
        swa_bytes = B * ATTN_NKV * ATTN_WINDOW * ATTN_D * 2 * 2
        step_bytes = 14 * kv_bytes + 35 * swa_bytes
        status = 0
        for L in layers:
            status |= _ws_status(moe, L["ws"])
        nonfinite = any(not torch.isfinite(L["o"].view(torch.bfloat16).float()).all().item() for L in layers)
        full_gbs = kv_bytes / (full_us * 1e-6) / 1e9
        out[f"b{B}"] = {
            "us_per_step": round(step_us, 2), "tokens_per_s": round(B * 1e6 / step_us, 1),
            "us_per_step_fused_layer": round(fused_us, 2), "fused_equals_prep_decode": fused_same,
            "step_GBps": round(step_bytes / (step_us * 1e-6) / 1e9, 1), "step_kv_bytes": int(step_bytes),
            "full_decode_us": round(full_us, 2), "full_decode_GBps": round(full_gbs, 1),
            "full_decode_hbm_frac": round(full_gbs / HBM_PEAK_GBS, 4), "full_decode_kv_bytes": int(kv_bytes),
            "context_positions": span, "status": status, "nonfinite": nonfinite,
            "layers": "14 full-context (no RoPE) + 35 window-513 (RoPE), prep + decode each"}
        log(f"attention B={B}: {step_us:.1f} us per 49-layer step (fused layer calls {fused_us:.1f} us, equal "
            f"{fused_same}), full-context decode {full_us:.1f} us ({full_gbs:.0f} GB/s), status {status}")
        del layers, g
        torch.cuda.empty_cache()
    return out


def _ws_status(moe, ws):
    import torch
    s = torch.full((1,), -1, dtype=torch.int32, device=ws.device)
    moe.moe_decode_wait_status(ws, s)
    return int(s.item())


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

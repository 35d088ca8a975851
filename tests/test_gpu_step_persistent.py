"""GPU tests of the persistent decode step (moe_decode_step_persistent),
through the C ABI: on every stack it must give moe_decode_step's output bit
for bit (same arithmetic and reduction orders; moe_decode_step is gated
against the oracle layer by layer in test_gpu_step.py), on a workspace that
starts as garbage, on a second call, across launches of up to 24 layers, at
run boundaries (dense layers, shape changes) and under HIP-graph replays."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import from_dev_bits, log, to_dev_bits, wait_status

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402

SMALL = dict(hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6)


def layers_of(kind):
    if kind == "small":
        dense = [synth.make_layer(100 + i, hidden=256, inter=0, shared_inter=256, n_experts=0, norm=True,
                                  residual=True) for i in range(2)]
        return dense + [synth.make_layer(110 + i, bias="zipf", norm=True, residual=True, **SMALL) for i in range(3)]
    if kind == "mixed":
        a = synth.make_layer(121, bias="zipf", norm=True, residual=True, **SMALL)
        b = synth.make_layer(122, bias="zipf", norm=True, residual=True, hidden=256, inter=128, shared_inter=128,
                             n_experts=64, top_k=8)
        d = synth.make_layer(120, hidden=256, inter=0, shared_inter=256, n_experts=0, norm=True, residual=True)
        return [a, a, d, b, b, b, a]
    if kind == "long":  # two launches (24 + 13 layers) of 5 distinct small layers
        base = [synth.make_layer(130 + i, bias="zipf", norm=True, residual=True, **SMALL) for i in range(5)]
        return [base[i % 5] for i in range(37)]
    if kind == "nonorm":
        return [synth.make_layer(140 + i, residual=True, **SMALL) for i in range(4)]
    # the model's shapes: 2 dense (intermediate 5632) + MoE layers
    dense = [synth.make_layer(i, inter=0, shared_inter=5632, n_experts=0, norm=True, residual=True) for i in range(2)]
    return dense + [synth.make_layer(2 + i, norm=True, residual=True) for i in range(6)]


def setup(kind):
    layers = layers_of(kind)
    cache = {}
    devs = []
    for L in layers:  # repeated layer dicts share one device copy
        if id(L) not in cache:
            cache[id(L)] = moe.DeviceLayer(L)
        devs.append(cache[id(L)])
    return layers, devs, [d.desc for d in devs], [d.weights for d in devs]


@pytest.mark.parametrize("kind,B", [("small", 1), ("mixed", 1), ("long", 1), ("nonorm", 1), ("full", 1),
                                    ("small", 3), ("full", 8)])
def test_persistent_step_equals_step(kind, B):
    log(f"test: persistent step {kind} B={B}")
    layers, devs, descs, ws_ = setup(kind)
    H = layers[0]["hidden"]
    x = to_dev_bits(synth.tokens(B, H, stream=900 + B))
    y_ref = torch.empty_like(x)
    ws_s = torch.zeros(moe.moe_decode_step_workspace_bytes(descs, B), dtype=torch.uint8, device="cuda")
    moe.moe_decode_step(descs, ws_, x, B, y_ref, ws_s, ws_s.numel())
    nbytes = moe.moe_decode_step_persistent_workspace_bytes(descs, B)
    assert nbytes > ws_s.numel()
    ws_p = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")   # garbage to start with
    y = torch.empty_like(x)
    moe.moe_decode_step_persistent(descs, ws_, x, B, y, ws_p, nbytes)
    torch.cuda.synchronize()
    assert wait_status(ws_s) == 0 and wait_status(ws_p) == 0
    assert np.array_equal(from_dev_bits(y), from_dev_bits(y_ref))
    # again on the same workspace, with another token
    x2 = to_dev_bits(synth.tokens(B, H, stream=950 + B))
    moe.moe_decode_step(descs, ws_, x2, B, y_ref, ws_s, ws_s.numel())
    moe.moe_decode_step_persistent(descs, ws_, x2, B, y, ws_p, nbytes)
    torch.cuda.synchronize()
    assert wait_status(ws_p) == 0
    assert np.array_equal(from_dev_bits(y), from_dev_bits(y_ref))


def test_persistent_step_too_small_workspace():
    _, _, descs, ws_ = setup("small")
    x = to_dev_bits(synth.tokens(1, 256, stream=901))
    y = torch.empty_like(x)
    n = moe.moe_decode_step_workspace_bytes(descs, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_step_persistent(descs, ws_, x, 1, y, ws, n)
    assert e.value.status == moe.MOE_ERR_WORKSPACE


def test_persistent_step_graph_replays():
    # one captured persistent step replayed with a new token each time,
    # each replay equal to an eager moe_decode_step
    log("test: persistent step graph replays")
    layers, devs, descs, ws_ = setup("full")
    H = layers[0]["hidden"]
    x = to_dev_bits(synth.tokens(1, H, stream=960))
    y = torch.empty_like(x)
    nbytes = moe.moe_decode_step_persistent_workspace_bytes(descs, 1)
    ws_p = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    ws_s = torch.zeros(moe.moe_decode_step_workspace_bytes(descs, 1), dtype=torch.uint8, device="cuda")
    y_ref = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_decode_step_persistent(descs, ws_, x, 1, y, ws_p, nbytes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_decode_step_persistent(descs, ws_, x, 1, y, ws_p, nbytes)
    for r in range(3):
        x.copy_(to_dev_bits(synth.tokens(1, H, stream=961 + r)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out = from_dev_bits(y).copy()
        assert wait_status(ws_p) == 0
        moe.moe_decode_step(descs, ws_, x, 1, y_ref, ws_s, ws_s.numel())
        torch.cuda.synchronize()
        assert np.array_equal(out, from_dev_bits(y_ref)), r

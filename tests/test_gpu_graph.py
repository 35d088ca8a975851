"""HIP-graph replays of the decode step through the C ABI.  The step's
kernels hand values between their blocks through tagged sync words that
every call zeroes first; a captured step must give, on every replay, the
bits the same step gives when enqueued eagerly, also with eager calls on
the graph's own workspace between the replays and a new token each time."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import log, to_dev_bits, wait_status

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402

H = 256


def layers():
    kw = dict(hidden=H, inter=64, shared_inter=64, n_experts=32, top_k=6)
    return [synth.make_layer(140, bias="zipf", norm=True, residual=True, **kw),
            synth.make_layer(141, hidden=H, inter=0, shared_inter=256, n_experts=0, norm=True, residual=True),
            synth.make_layer(142, norm=True, residual=True, **kw)]


@pytest.mark.parametrize("B", [1, 3, 16])
def test_graph_replays_match_eager_calls(B):
    log(f"test: graph replays B={B}")
    devs = [moe.DeviceLayer(L) for L in layers()]
    descs = [d.desc for d in devs]
    wts = [d.weights for d in devs]
    n = moe.moe_decode_step_workspace_bytes(descs, B)
    ws = torch.full((n,), 255, dtype=torch.uint8, device="cuda")  # starts as garbage
    ws_eager = torch.zeros(n, dtype=torch.uint8, device="cuda")
    x = to_dev_bits(synth.tokens(B, H, stream=900))
    y = torch.empty_like(x)

    def eager(xin, wsp):
        out = torch.empty_like(xin)
        moe.moe_decode_step(descs, wts, xin, B, out, wsp, wsp.numel())
        torch.cuda.synchronize()
        return out

    moe.moe_decode_step(descs, wts, x, B, y, ws, ws.numel())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_decode_step(descs, wts, x, B, y, ws, ws.numel())
    torch.cuda.synchronize()
    for i in range(4):
        xi = to_dev_bits(synth.tokens(B, H, stream=910 + i))
        x.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        assert wait_status(ws) == 0, f"replay {i}"
        ref = eager(xi, ws_eager)
        assert wait_status(ws_eager) == 0
        assert torch.equal(y, ref), f"replay {i}"
        assert np.all(np.isfinite(y.view(torch.bfloat16).float().cpu().numpy()))
        # eager work on the graph's own workspace between the replays
        assert torch.equal(eager(xi, ws), ref), f"eager on the graph workspace {i}"
        assert wait_status(ws) == 0

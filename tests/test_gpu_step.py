"""GPU parity of the multi-layer decode step (dense layers then MoE layers,
pre-norm residual blocks) through the C ABI: each GPU layer fed the
oracle's input to that layer must pass the layer bar on its own output o
(residual add off: on a residual stream with |x| >= 2 one BF16 ulp is
0.0156, above the 1e-2 max-abs bar, so x + o is checked separately and
exactly); the step must equal the chain of single-layer calls bit for bit;
end-to-end drift over the stack is reported."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_f64, compare, from_dev_bits, log, to_dev_bits, wait_status

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402


def stack(kind):
    if kind == "small":
        kw = dict(hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6)
        dense = [synth.make_layer(100 + i, hidden=256, inter=0, shared_inter=256, n_experts=0, norm=True,
                                  residual=True) for i in range(2)]
        moes = [synth.make_layer(110 + i, bias="zipf", norm=True, residual=True, **kw) for i in range(3)]
    elif kind == "mixed":
        # MoE layers of different shapes in one step (their one-token sync
        # words share one region of the workspace), a dense layer between
        dense = [synth.make_layer(120, hidden=256, inter=0, shared_inter=256, n_experts=0, norm=True,
                                  residual=True)]
        moes = [synth.make_layer(121, bias="zipf", norm=True, residual=True, hidden=256, inter=64,
                                 shared_inter=64, n_experts=32, top_k=6),
                synth.make_layer(122, bias="zipf", norm=True, residual=True, hidden=256, inter=128,
                                 shared_inter=128, n_experts=64, top_k=8),
                synth.make_layer(123, norm=True, residual=True, hidden=256, inter=64, shared_inter=0,
                                 n_experts=16, top_k=2)]
        return [moes[0], dense[0], moes[1], moes[2], moes[0]]
    else:  # the model's shapes: 2 dense (intermediate 5632) + MoE layers
        dense = [synth.make_layer(i, inter=0, shared_inter=5632, n_experts=0, norm=True, residual=True)
                 for i in range(2)]
        moes = [synth.make_layer(2 + i, norm=True, residual=True) for i in range(4)]
    return dense + moes


@pytest.mark.parametrize("kind,B", [("small", 1), ("small", 8), ("mixed", 1), ("mixed", 3), ("full", 1),
                                    ("full", 8), ("full", 16)])
def test_step_matches_layers_and_oracle(kind, B):
    log(f"test: step {kind} B={B}")
    layers = stack(kind)
    H = layers[0]["hidden"]
    devs = [moe.DeviceLayer(L) for L in layers]
    descs = [d.desc for d in devs]
    ws_ = [d.weights for d in devs]
    x = synth.tokens(B, H, stream=700 + B)
    xt = to_dev_bits(x)
    y = torch.empty_like(xt)
    ws = torch.zeros(moe.moe_decode_step_workspace_bytes(descs, B), dtype=torch.uint8, device="cuda")
    moe.moe_decode_step(descs, ws_, xt, B, y, ws, ws.numel())
    assert wait_status(ws) == 0
    # a second call on the same workspace (which now holds the first call's
    # sync words) gives the same bits
    y2 = torch.empty_like(xt)
    moe.moe_decode_step(descs, ws_, xt, B, y2, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert wait_status(ws) == 0
    # the same layers one call at a time
    cur = xt
    for d in devs:
        cur, _, _ = d.decode(cur)
        assert d.wait_status() == 0
    step_out = from_dev_bits(y)
    assert np.array_equal(step_out, from_dev_bits(cur))
    # per layer against the oracle, each fed the oracle's own input
    xo = x
    for i, (L, d) in enumerate(zip(layers, devs)):
        o, idx, w = d.decode(to_dev_bits(xo), residual=0)
        assert d.wait_status() == 0
        yr, _, _ = d.decode(to_dev_bits(xo), residual=1)
        torch.cuda.synchronize()
        assert d.wait_status() == 0
        k = L["top_k"] if L["n_experts"] else 0
        o = from_dev_bits(o)
        compare(dict(L, residual=0), xo, o, idx.cpu().numpy()[:, :k], w.cpu().numpy()[:, :k],
                what=f"{kind} layer {i} B={B}")
        # the residual add: one BF16 rounding of x + o
        want = np.array([oracle.bf16_round(v) for v in (bf16_f64(xo) + bf16_f64(o)).ravel()],
                        np.uint16).reshape(o.shape)
        assert np.array_equal(from_dev_bits(yr), want)
        xo = oracle.moe_tokens(L, xo)["out"]
    o, r = bf16_f64(step_out), bf16_f64(xo)
    drift = float(np.linalg.norm(o - r) / np.linalg.norm(r))
    log(f"  end-to-end rel-L2 drift over {len(layers)} layers: {drift:.2e}")
    assert drift < 2e-2

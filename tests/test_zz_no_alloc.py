"""The entry point that allocates nothing (moe_decode_layer_noalloc): its
workspace is the library's per-GPU device array.  Through the C ABI, two
calls in a row (the full 256-expert layer at batch 8, then a smaller layer
at batch 3, which finds the first call's contents in the array) must each
give the bits moe_decode_layer gives on a workspace of its own, and pass
the oracle's acceptance bar; the array's wait status must read zero."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import compare, from_dev_bits, log, to_dev_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402


def _both(L, dev, B, stream_id):
    x = synth.tokens(B, L["hidden"], stream=stream_id)
    xt = to_dev_bits(x)
    k = L["top_k"]
    outs = []
    for which in ("noalloc", "ws"):
        y = torch.empty_like(xt)
        idx = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
        w = torch.zeros((B, k), dtype=torch.float32, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        if which == "noalloc":
            moe.moe_decode_layer_noalloc(dev.desc, dev.weights, xt, B, 0, y, idx, w)
            moe.moe_decode_wait_status(None, st)
        else:
            ws = torch.full((moe.moe_decode_workspace_bytes(dev.desc, B),), 255, dtype=torch.uint8, device="cuda")
            moe.moe_decode_layer(dev.desc, dev.weights, xt, B, 0, y, idx, w, ws, ws.numel())
            moe.moe_decode_wait_status(ws, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, which
        outs.append((from_dev_bits(y), idx.cpu().numpy(), w.cpu().numpy()))
    return x, outs


def test_noalloc_matches_workspace_entry_point_twice():
    layers = [(synth.make_layer(0, wtype="nvfp4", bias="zipf"), 8, 61),
              (synth.make_layer(22, hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6, bias="zipf",
                                norm=True), 3, 62)]
    for i, (L, B, sid) in enumerate(layers):
        log(f"test: no-alloc call {i}: H={L['hidden']} E={L['n_experts']} B={B}")
        dev = moe.DeviceLayer(L)
        assert moe.moe_decode_workspace_bytes(dev.desc, B) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        x, ((o0, i0, w0), (o1, i1, w1)) = _both(L, dev, B, sid)
        assert np.array_equal(o0, o1) and np.array_equal(i0, i1) and np.array_equal(w0, w1), f"call {i}"
        _, st = compare(L, x, o0, i0, w0, what=f"no-alloc call {i}")
        log(f"  {st}")

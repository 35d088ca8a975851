"""GPU parity of the dense NVFP4 projection (moe_gemv_nvfp4) against the
CPU oracle, through the C ABI: shapes of the projections outside the MoE
blocks (attention QKV and output from 32 query and 4 KV heads of 128, an
LM-head slice whose vocabulary the pages do not give) and ragged ones,
batches 1..8."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_outputs, from_dev_bits, log, to_dev_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402


def _matrix(rows, cols, seed):
    m, s = synth.nvfp4_stack(seed, 0, 1, 1, rows, cols)
    src = torch.from_numpy(m.reshape(-1)).cuda()
    w = torch.empty_like(src)
    moe.moe_repack_nvfp4(src, w, rows, cols, 1)
    return m[0], float(s[0]), w, torch.tensor([s[0]], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("rows,cols,B", [
    (8, 64, 1), (24, 128, 3), (264, 2112, 2),          # ragged: last block partly filled; 66 chunks per row
    (5120, 2048, 1), (5120, 2048, 8),                  # fused QKV: (32 query + 4 + 4 KV heads) x 128
    (2048, 4096, 5), (2048, 4096, 1),                  # attention output: 32 heads x 128 in
    (2048, 5632, 1), (5632, 2048, 4),                  # dense MLP shapes
    (16384, 2048, 1), (16384, 2048, 8),                # an LM-head slice
    (256, 4096, 8), (512, 5632, 3),                    # batch x cols above the LDS stage: x from memory
])
def test_gemv_matches_oracle(rows, cols, B):
    log(f"test: gemv {rows}x{cols} B={B}")
    src, S, w, s = _matrix(rows, cols, rows + cols + B)
    x = synth.tokens(B, cols, stream=rows + B)
    y = torch.empty((B, rows), dtype=torch.int16, device="cuda")
    moe.moe_gemv_nvfp4(w, s, rows, cols, to_dev_bits(x), B, y)
    torch.cuda.synchronize()
    ref, nan = oracle.gemv_nvfp4(src, rows, cols, S, x)
    assert nan == 0
    st = check_outputs(from_dev_bits(y), ref, f"gemv {rows}x{cols} B={B}")
    log(f"  {st}")


def test_gemv_batch_rows_independent_and_deterministic():
    # each token's row of y depends on that token alone, bit for bit
    rows, cols = 1024, 2048
    src, S, w, s = _matrix(rows, cols, 77)
    x = synth.tokens(8, cols, stream=77)
    xt = to_dev_bits(x)
    y8 = torch.empty((8, rows), dtype=torch.int16, device="cuda")
    moe.moe_gemv_nvfp4(w, s, rows, cols, xt, 8, y8)
    for B in (1, 3):
        yb = torch.empty((B, rows), dtype=torch.int16, device="cuda")
        moe.moe_gemv_nvfp4(w, s, rows, cols, xt[2:2 + B].contiguous(), B, yb)
        torch.cuda.synchronize()
        assert torch.equal(yb, y8[2:2 + B])
    y8b = torch.empty_like(y8)
    moe.moe_gemv_nvfp4(w, s, rows, cols, xt, 8, y8b)
    torch.cuda.synchronize()
    assert torch.equal(y8, y8b)


def test_gemv_zero_input_and_constant_code():
    rows, cols = 64, 256
    blk = np.array([0x38] + [0x22] * 8, np.uint8)  # scale 1.0, every code 2 (= 1.0)
    m = np.tile(blk, (rows, cols // 16))
    src = torch.from_numpy(m.reshape(-1)).cuda()
    w = torch.empty_like(src)
    moe.moe_repack_nvfp4(src, w, rows, cols, 1)
    s = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    x = synth.tokens(2, cols, stream=5)
    x[1] = 0
    y = torch.empty((2, rows), dtype=torch.int16, device="cuda")
    moe.moe_gemv_nvfp4(w, s, rows, cols, to_dev_bits(x), 2, y)
    torch.cuda.synchronize()
    ref, _ = oracle.gemv_nvfp4(m, rows, cols, 0.5, x)
    out = from_dev_bits(y)
    assert np.all(out[1] == 0) and np.all(out[0] == out[0, 0])
    check_outputs(out, ref, "constant code")

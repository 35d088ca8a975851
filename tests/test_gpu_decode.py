"""GPU parity of the decode path (and the repack) against the CPU oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import compare, from_dev_bits, log, to_dev_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402


def run(layer, x, dev=None, ws=None):
    dev = dev or moe.DeviceLayer(layer)
    y, idx, w = dev.decode(to_dev_bits(x), ws=ws)
    torch.cuda.synchronize()
    assert dev.wait_status() == 0
    k = layer["top_k"] if layer["n_experts"] else 0
    return from_dev_bits(y), idx.cpu().numpy()[:, :k], w.cpu().numpy()[:, :k]


# ---------------------------------------------------------------- repack


def _code_matrix():
    # Row s: block 0 = scale code s with element codes 0..15, block 1 =
    # scale code s with element codes 15..0 (every E2M1 x E4M3 pair, twice).
    rows = []
    for s in range(256):
        b0 = [s] + [j | ((j + 8) << 4) for j in range(8)]
        b1 = [s] + [(15 - j) | ((7 - j) << 4) for j in range(8)]
        rows.append(b0 + b1)
    return np.array(rows, dtype=np.uint8)


def test_every_e2m1_x_e4m3_code_through_repack_and_dequant():
    log("test: all 16x256 codes")
    src = _code_matrix()  # [256 rows][32 cols] -> 2 blocks of 9 bytes per row
    s = torch.from_numpy(src.reshape(-1)).cuda()
    d = torch.empty_like(s)
    nan = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_repack_nvfp4(s, d, 256, 32, 1, nan)
    back = torch.empty_like(s)
    moe.moe_unpack_nvfp4(d, back, 256, 32, 1)
    vals = torch.empty((256, 32), dtype=torch.float32, device="cuda")
    sc = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    moe.moe_dequant_nvfp4(d, vals, 256, 32, 1, sc)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), src.reshape(-1))
    assert int(nan.item()) == 4  # codes 0x7F and 0xFF, two blocks each
    ref, n_nan = oracle.decode_nvfp4(src, 256, 32, 0.5)
    assert n_nan == 4
    got = vals.cpu().numpy().astype(np.float64)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, ref))
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


@pytest.mark.parametrize("rows,cols,n", [(8, 32, 1), (16, 64, 3), (512, 2048, 2), (2048, 512, 1), (40, 5632, 1)])
def test_repack_round_trip_random_bytes(rows, cols, n):
    log(f"test: repack round trip {rows}x{cols}x{n}")
    rng = np.random.default_rng(rows * 7 + cols + n)
    src = rng.integers(0, 256, size=n * rows * cols * 9 // 16, dtype=np.uint8)
    s = torch.from_numpy(src).cuda()
    d = torch.empty_like(s)
    nan = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_repack_nvfp4(s, d, rows, cols, n, nan)
    back = torch.empty_like(s)
    moe.moe_unpack_nvfp4(d, back, rows, cols, n)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), src)
    scales = src.reshape(-1, 9)[:, 0]
    assert int(nan.item()) == int(np.sum((scales & 0x7F) == 0x7F))
    # the repacked bytes decode to the same values as the source
    ref, _ = oracle.decode_nvfp4(src[: rows * cols * 9 // 16], rows, cols, 1.0)
    vals = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    moe.moe_dequant_nvfp4(d, vals, rows, cols, 1)
    got = vals.cpu().numpy().astype(np.float64)
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m]) and np.all(np.isnan(got[~m]))


# ---------------------------------------------------------------- small shapes

SMALL = dict(hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6)


@pytest.mark.parametrize("wtype", ["nvfp4", "bf16"])
@pytest.mark.parametrize("B", [1, 2, 5, 8])
def test_decode_small(wtype, B):
    log(f"test: decode small {wtype} B={B}")
    L = synth.make_layer(11, wtype=wtype, bias="zipf", **SMALL)
    x = synth.tokens(B, 256, stream=100 + B)
    out, idx, w = run(L, x)
    _, st = compare(L, x, out, idx, w, what=f"small {wtype} B={B}")
    log(f"  {st}")


@pytest.mark.parametrize("B", [9, 12, 16])
def test_decode_small_sixteen_token_batches(B):
    # NVFP4 batches of 9..16 tokens: the tokens fill the 16 columns of the
    # gate/up tiles and two token groups of the down tiles.
    log(f"test: decode small nvfp4 B={B}")
    L = synth.make_layer(11, bias="zipf", **SMALL)
    x = synth.tokens(B, 256, stream=100 + B)
    out, idx, w = run(L, x)
    _, st = compare(L, x, out, idx, w, what=f"small nvfp4 B={B}")
    log(f"  {st}")


@pytest.mark.parametrize("B", [1, 8, 16])
def test_decode_small_norm_residual(B):
    log(f"test: decode small norm+residual B={B}")
    L = synth.make_layer(12, bias="zipf", norm=True, residual=True, **SMALL)
    x = synth.tokens(B, 256, stream=200 + B)
    out, idx, w = run(L, x)
    compare(L, x, out, idx, w, what="norm+residual")


def test_decode_all_experts_selected():
    L = synth.make_layer(13, hidden=128, inter=64, shared_inter=64, n_experts=8, top_k=8)
    x = synth.tokens(3, 128, stream=5)
    out, idx, w = run(L, x)
    assert all(sorted(r) == list(range(8)) for r in idx.tolist())
    compare(L, x, out, idx, w, what="k=E")


def test_decode_top1_no_shared():
    L = synth.make_layer(14, hidden=128, inter=64, shared_inter=0, n_experts=16, top_k=1)
    x = synth.tokens(4, 128, stream=6)
    out, idx, w = run(L, x)
    assert np.all(w == 1.0)
    compare(L, x, out, idx, w, what="k=1, no shared")


@pytest.mark.parametrize("B", [8, 16])
def test_decode_identical_tokens_share_experts(B):
    L = synth.make_layer(15, **SMALL)
    x = np.repeat(synth.tokens(1, 256, stream=7), B, axis=0)
    out, idx, w = run(L, x)
    assert len({tuple(sorted(r)) for r in idx.tolist()}) == 1
    assert np.all(out == out[0:1])
    compare(L, x, out, idx, w, what="identical tokens")


def test_decode_zero_input_full_tie():
    L = synth.make_layer(16, **SMALL)
    x = np.zeros((2, 256), np.uint16)
    out, idx, w = run(L, x)
    assert np.all(idx == np.arange(6)) and np.all(out == 0)


@pytest.mark.parametrize("E,B", [(32, 1), (1000, 1), (1000, 3)])
def test_decode_zero_input_full_tie_any_width(E, B):
    # Every logit equal (zero input, zero bias): the k lowest expert indices
    # in order, through the one-token kernel (B = 1) and the batch routing,
    # with 4 and 16 logits per lane in the top-k.
    L = synth.make_layer(20, hidden=256, inter=64, shared_inter=64, n_experts=E, top_k=6)
    x = np.zeros((B, 256), np.uint16)
    out, idx, w = run(L, x)
    assert np.all(idx == np.arange(6)) and np.all(out == 0)


@pytest.mark.parametrize("E,B", [(512, 1), (1000, 1), (1000, 5)])
def test_decode_many_experts(E, B):
    # More than 256 experts: the top-k holds 16 logits per lane, and 1000
    # leaves the last lanes partly empty.
    log(f"test: decode many experts E={E} B={B}")
    L = synth.make_layer(19, hidden=256, inter=64, shared_inter=64, n_experts=E, top_k=8, bias="zipf")
    x = synth.tokens(B, 256, stream=19 + B)
    out, idx, w = run(L, x)
    compare(L, x, out, idx, w, what=f"E={E} B={B}")


@pytest.mark.parametrize("B,norm", [(8, False), (8, True), (1, True)])
def test_decode_wide_hidden_multi_chunk_lanes(B, norm):
    # H = 4096: 128 chunks per row, two per lane; with the pre-norm, each
    # norm or router thread takes two 16-byte pieces of every token.  The
    # residual stays off: the bar applies to the layer output alone.
    L = synth.make_layer(17, hidden=4096, inter=128, shared_inter=128, n_experts=16, top_k=4, bias="zipf",
                         norm=norm)
    x = synth.tokens(B, 4096, stream=9)
    out, idx, w = run(L, x)
    compare(L, x, out, idx, w, what=f"H=4096 B={B} norm={norm}")


@pytest.mark.parametrize("Is,norm,B", [(2112, True, 2), (2112, False, 2), (256, True, 2), (2112, True, 16),
                                        (256, False, 11)])
def test_dense_layer_small(Is, norm, B):
    # 2112 = 66 chunks of 32: two chunk steps per lane, the second ragged
    # (and five K pieces per entry in the batch down kernel).
    L = synth.make_layer(18, hidden=256, inter=0, shared_inter=Is, n_experts=0, norm=norm, residual=norm)
    x = synth.tokens(B, 256, stream=10)
    out, _, _ = run(L, x)
    compare(L, x, out, None, None, what=f"dense B={B}")


def test_workspace_reuse_across_batches_and_determinism():
    L = synth.make_layer(19, bias="zipf", **SMALL)
    dev = moe.DeviceLayer(L)
    ws = dev.workspace(16)
    for B in (8, 1, 16, 3, 9, 8):
        x = synth.tokens(B, 256, stream=300 + B)
        a = run(L, x, dev, ws)
        b = run(L, x, dev, ws)
        assert all(np.array_equal(u, v) for u, v in zip(a, b)), B
        compare(L, x, *a, what=f"reuse B={B}")


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_one_token_handover_garbage_workspace_changing_inputs(fill):
    # One token: the expert kernel hands h from its gate/up blocks to its
    # down blocks through the workspace (words, per-XCD tickets, flags and
    # copies).  A workspace that starts as garbage, and back-to-back calls
    # with different tokens and layers (so stale data from the previous call
    # would be wrong), must each give that call's own result.
    L1 = synth.make_layer(20, bias="zipf", norm=True, **SMALL)
    L2 = synth.make_layer(21, **SMALL)
    d1, d2 = moe.DeviceLayer(L1), moe.DeviceLayer(L2)
    n = max(moe.moe_decode_workspace_bytes(d.desc, 8) for d in (d1, d2))
    if fill == "ones":
        ws = torch.full((n,), 255, dtype=torch.uint8, device="cuda")
    else:
        g = torch.Generator(device="cpu").manual_seed(5)
        ws = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
    seq = [(L1, d1, 1), (L2, d2, 1), (L1, d1, 8), (L1, d1, 1), (L2, d2, 1), (L2, d2, 3), (L1, d1, 1)]
    for i, (L, d, B) in enumerate(seq):
        x = synth.tokens(B, 256, stream=800 + i)
        out, idx, w = run(L, x, d, ws)
        compare(L, x, out, idx, w, what=f"hand-over {fill} call {i} B={B}")


# ---------------------------------------------------------------- full shapes

_cache = {}


def full_layer(kind):
    if kind not in _cache:
        log(f"generating full layer {kind}")
        if kind == "bf16":
            _cache[kind] = synth.make_layer(0, wtype="bf16")
        elif kind == "nvfp4":
            _cache[kind] = synth.make_layer(0, wtype="nvfp4")
        elif kind == "zipf":
            _cache[kind] = synth.make_layer(0, wtype="nvfp4", bias="zipf")
        elif kind == "norm":
            _cache[kind] = synth.make_layer(2, wtype="nvfp4", bias="zipf", norm=True, residual=True)
        elif kind == "dense":
            _cache[kind] = synth.make_layer(0, inter=0, shared_inter=5632, n_experts=0, norm=True, residual=True)
    return _cache[kind]


@pytest.mark.parametrize("kind,B", [("bf16", 1), ("nvfp4", 1), ("zipf", 8), ("nvfp4", 8), ("norm", 1),
                                    ("norm", 8), ("dense", 1), ("zipf", 16), ("nvfp4", 12), ("dense", 16)])
def test_decode_full_shape(kind, B):
    log(f"test: full shape {kind} B={B}")
    L = full_layer(kind)
    x = synth.tokens(B, 2048, stream=400 + B)
    out, idx, w = run(L, x)
    _, st = compare(L, x, out, idx, w, what=f"full {kind} B={B}")
    if L["n_experts"]:
        st["distinct"] = len(np.unique(idx))
    log(f"  {st}")

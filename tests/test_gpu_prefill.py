"""GPU parity of the prefill path (tokens grouped by expert, matrix-core
GEMMs) against the CPU oracle, through the C ABI.  Each token's result is
independent of the others; the oracle runs the tokens over every host
thread, so even the full 8192-token shape is checked token by token."""
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


def run(layer, x, dev=None, ws=None, residual=None):
    dev = dev or moe.DeviceLayer(layer)
    y, idx, w = dev.prefill(to_dev_bits(x), ws=ws, residual=residual)
    torch.cuda.synchronize()
    k = layer["top_k"] if layer["n_experts"] else 0
    return from_dev_bits(y), idx.cpu().numpy()[:, :k], w.cpu().numpy()[:, :k]


def check_routing_properties(layer, idx, w):
    E, k = layer["n_experts"], layer["top_k"]
    assert idx.min() >= 0 and idx.max() < E
    assert all(len(set(r)) == k for r in idx.tolist())
    assert np.all(w > 0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=2e-6)


SMALL = dict(hidden=256, inter=64, shared_inter=64, n_experts=16, top_k=4)


@pytest.mark.parametrize("wtype", ["nvfp4", "bf16"])
@pytest.mark.parametrize("T", [1, 37, 300, 1000, 1024, 1025])
def test_prefill_small(wtype, T):
    # zipf bias: the favoured experts get several tiles with a ragged last
    # tile.  NVFP4 calls of 49..1024 tokens run 32-row tiles (T = 1024 is
    # the last), longer ones 128-row tiles (T = 1025 the first: the shared
    # expert's 9th tile holds 1 row); BF16 calls always 128-row tiles.
    log(f"test: prefill small {wtype} T={T}")
    L = synth.make_layer(31, wtype=wtype, bias="zipf", **SMALL)
    x = synth.tokens(T, 256, stream=500 + T)
    out, idx, w = run(L, x)
    check_routing_properties(L, idx, w)
    _, st = compare(L, x, out, idx, w, what=f"prefill small {wtype} T={T}")
    counts = np.bincount(idx.reshape(-1), minlength=L["n_experts"])
    st["max_rows_per_expert"] = int(counts.max())
    log(f"  {st}")


@pytest.mark.parametrize("T", [5, 257])
def test_prefill_norm_residual(T):
    L = synth.make_layer(32, bias="zipf", norm=True, residual=True, **SMALL)
    x = synth.tokens(T, 256, stream=600 + T)
    out, idx, w = run(L, x)
    compare(L, x, out, idx, w, what=f"prefill norm+residual T={T}")


def test_prefill_ragged_columns_and_depth():
    # H = 2112 (66 chunks): the down GEMM's last 128-column block holds 64
    # columns; I = 2080 (65 chunks): the gate/up GEMM's last 64-column block
    # holds 32 columns and the down GEMM's depth is not a multiple of 64.
    L = synth.make_layer(33, hidden=2112, inter=2080, shared_inter=2080, n_experts=8, top_k=2, bias="zipf")
    x = synth.tokens(150, 2112, stream=7)
    out, idx, w = run(L, x)
    compare(L, x, out, idx, w, what="ragged columns")


def test_prefill_all_experts_selected():
    L = synth.make_layer(34, hidden=128, inter=64, shared_inter=64, n_experts=8, top_k=8)
    x = synth.tokens(130, 128, stream=8)
    out, idx, w = run(L, x)
    assert all(sorted(r) == list(range(8)) for r in idx.tolist())
    compare(L, x, out, idx, w, what="k=E")


def test_prefill_top1_no_shared():
    L = synth.make_layer(35, hidden=128, inter=64, shared_inter=0, n_experts=16, top_k=1)
    x = synth.tokens(77, 128, stream=9)
    out, idx, w = run(L, x)
    assert np.all(w == 1.0)
    compare(L, x, out, idx, w, what="k=1, no shared")


def test_prefill_identical_tokens_one_expert_set():
    # All 600 tokens pick the same k experts: each of them gets 600 rows
    # (five 128-row tiles), every other expert none.
    L = synth.make_layer(36, **SMALL)
    x = np.repeat(synth.tokens(1, 256, stream=10), 600, axis=0)
    out, idx, w = run(L, x)
    assert len({tuple(sorted(r)) for r in idx.tolist()}) == 1
    assert np.all(out == out[0:1])
    compare(L, x[:3], out[:3], idx[:3], w[:3], what="identical tokens")


def test_prefill_zero_input_full_tie():
    L = synth.make_layer(37, **SMALL)
    x = np.zeros((50, 256), np.uint16)
    out, idx, w = run(L, x)
    assert np.all(idx == np.arange(4)) and np.all(out == 0)


@pytest.mark.parametrize("Is,norm", [(2112, True), (256, False)])
def test_prefill_dense_layer(Is, norm):
    L = synth.make_layer(38, hidden=256, inter=0, shared_inter=Is, n_experts=0, norm=norm, residual=norm)
    x = synth.tokens(200, 256, stream=11)
    out, _, _ = run(L, x)
    compare(L, x, out, None, None, what="dense prefill")


def test_prefill_matches_decode_routing_and_workspace_reuse():
    # The same tokens through both paths select the same experts (the
    # oracle checks each path's values), and one prefill workspace serves a
    # larger and then a smaller call.
    L = synth.make_layer(39, bias="zipf", norm=True, **SMALL)
    dev = moe.DeviceLayer(L)
    ws = torch.zeros(moe.moe_prefill_workspace_bytes(dev.desc, 700), dtype=torch.uint8, device="cuda")
    for T in (700, 40):
        x = synth.tokens(T, 256, stream=700 + T)
        a = run(L, x, dev, ws)
        b = run(L, x, dev, ws)
        assert all(np.array_equal(u, v) for u, v in zip(a, b)), T
        ref, _ = compare(L, x, *a, what=f"reuse T={T}")
        for t0 in range(0, min(T, 64), 8):
            yd, idd, _ = dev.decode(to_dev_bits(x[t0:t0 + 8]))
            torch.cuda.synchronize()
            for t in range(8):
                if not ref["flag"][t0 + t]:
                    assert set(idd.cpu().numpy()[t].tolist()) == set(a[1][t0 + t].tolist())


def test_prefill_many_experts():
    # 1000 experts: the top-k holds 16 logits per lane (the last lanes partly
    # empty), and the router's column tiles end ragged.
    log("test: prefill many experts E=1000")
    L = synth.make_layer(21, hidden=256, inter=64, shared_inter=64, n_experts=1000, top_k=8, bias="zipf")
    x = synth.tokens(300, 256, stream=21)
    out, idx, w = run(L, x)
    check_routing_properties(L, idx, w)
    compare(L, x, out, idx, w, what="prefill E=1000")


def test_prefill_placement_second_pass():
    # 140,000 tokens x top-4 = 560,000 (token, k) pairs: more than the 1024
    # placement blocks take in one pass of 512 pairs each, so some blocks
    # place a second batch.  A token's result depends on that token alone,
    # so every token must match, bit for bit, the same tokens run in four
    # chunks that need one pass; a spread sample is checked by the oracle.
    T, chunks = 140_000, 4
    log(f"test: prefill placement second pass T={T}")
    L = synth.make_layer(13, **SMALL)
    dev = moe.DeviceLayer(L)
    x = synth.tokens(T, 256, stream=13)
    out, idx, w = run(L, x, dev)
    check_routing_properties(L, idx, w)
    n = T // chunks
    for c in range(chunks):
        oc, ic, wc = run(L, x[c * n:(c + 1) * n], dev)
        assert np.array_equal(ic, idx[c * n:(c + 1) * n]), f"chunk {c} experts"
        assert np.array_equal(wc, w[c * n:(c + 1) * n]), f"chunk {c} weights"
        assert np.array_equal(oc, out[c * n:(c + 1) * n]), f"chunk {c} outputs"
    s = sample_tokens(T, 64, 13)
    compare(L, x[s], out[s], idx[s], w[s], what=f"prefill second pass T={T}")


# Calls of up to 48 NVFP4 tokens run 16-row tiles (the small-tile kernels)
# and, with routed experts and H <= 16384, the per-token router that also
# clears the expert counts and cursors.
SMALL_TILE_CASES = {
    # 48 identical tokens: each of the 4 selected experts and the shared one
    # gets three full 16-row tiles
    "identical": (dict(SMALL), 48, "same"),
    # the last 64-column gate/up item holds 32 columns, the last 128-column
    # down item 64, and neither depth is a multiple of 128
    "ragged": (dict(hidden=2112, inter=2080, shared_inter=2080, n_experts=8, top_k=2, bias="zipf"), 40, None),
    "k_equals_E": (dict(hidden=128, inter=64, shared_inter=64, n_experts=8, top_k=8), 45, None),
    "top1_no_shared": (dict(hidden=128, inter=64, shared_inter=0, n_experts=16, top_k=1), 33, None),
    # 1000 experts: 250 router blocks per token, 1001 count and cursor words
    # cleared by the router's first block
    "many_experts": (dict(hidden=256, inter=64, shared_inter=64, n_experts=1000, top_k=8, bias="zipf"), 44, None),
    # no router: the pre-norm runs on its own, the shared expert in 16-row tiles
    "dense": (dict(hidden=256, inter=0, shared_inter=512, n_experts=0, norm=True), 20, None),
    # H = 16416 > 16384: the token does not fit the per-token router's LDS
    # stage, so the norm and the GEMM router run instead
    "wide_hidden": (dict(hidden=16416, inter=64, shared_inter=64, n_experts=4, top_k=2, norm=True, bias="zipf"), 3,
                    None),
}


@pytest.mark.parametrize("case", list(SMALL_TILE_CASES))
def test_prefill_small_tile_cases(case):
    kw, T, mode = SMALL_TILE_CASES[case]
    log(f"test: prefill small tiles {case} T={T}")
    L = synth.make_layer(41, wtype="nvfp4", **kw)
    H = kw["hidden"]
    if mode == "same":
        x = np.repeat(synth.tokens(1, H, stream=41), T, axis=0)
    else:
        x = synth.tokens(T, H, stream=41)
    out, idx, w = run(L, x)
    E = L["n_experts"]
    if E:
        check_routing_properties(L, idx, w)
    if mode == "same":
        assert len({tuple(sorted(r)) for r in idx.tolist()}) == 1
        assert np.all(out == out[0:1])
    compare(L, x, out, idx if E else None, w if E else None, what=f"small tiles {case}")


# Calls with fewer than 128 router tiles (64 tokens x 64 experts) split the
# router GEMM's depth (up to 8 ways); the top-k sums the partial logits.
# E % 4 != 0 takes the top-k's one-logit loads, E % 4 == 0 its 16-byte
# loads; 2048 deep gives the full 8 splits, 256 deep 2.
SPLIT_ROUTER_CASES = {
    "odd_E_2way": (dict(hidden=256, inter=64, shared_inter=64, n_experts=6, top_k=2, bias="zipf"), 100),
    "odd_E_8way": (dict(hidden=2048, inter=64, shared_inter=64, n_experts=6, top_k=2, bias="zipf"), 70),
    "E_multiple_of_4_8way": (dict(hidden=2048, inter=64, shared_inter=0, n_experts=20, top_k=3, norm=True), 130),
}


@pytest.mark.parametrize("case", list(SPLIT_ROUTER_CASES))
@pytest.mark.parametrize("wtype", ["nvfp4", "bf16"])
def test_prefill_split_router(case, wtype):
    kw, T = SPLIT_ROUTER_CASES[case]
    log(f"test: prefill split router {case} {wtype} T={T}")
    L = synth.make_layer(42, wtype=wtype, **kw)
    x = synth.tokens(T, kw["hidden"], stream=42)
    out, idx, w = run(L, x)
    check_routing_properties(L, idx, w)
    compare(L, x, out, idx, w, what=f"split router {case} {wtype}")


def test_prefill_rejects_and_sizes():
    L = synth.make_layer(40, **SMALL)
    dev = moe.DeviceLayer(L)
    assert moe.moe_prefill_workspace_bytes(dev.desc, 0) == 0
    n = moe.moe_prefill_workspace_bytes(dev.desc, 100)
    assert n > 0 and moe.moe_prefill_workspace_bytes(dev.desc, 200) > n
    ws = torch.zeros(n - 256, dtype=torch.uint8, device="cuda")
    x = to_dev_bits(synth.tokens(100, 256, stream=12))
    y = torch.empty_like(x)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_prefill_layer(dev.desc, dev.weights, x, 100, 0, y, None, None, ws, ws.numel())
    assert e.value.status == moe.MOE_ERR_WORKSPACE


# ---------------------------------------------------------------- full shape

_cache = {}


def full_layer(kind):
    if kind not in _cache:
        log(f"generating full layer {kind}")
        if kind == "norm":
            _cache[kind] = synth.make_layer(2, wtype="nvfp4", bias="zipf", norm=True, residual=True)
        elif kind == "nvfp4":
            _cache[kind] = synth.make_layer(0, wtype="nvfp4")
        elif kind == "dense":
            _cache[kind] = synth.make_layer(0, inter=0, shared_inter=5632, n_experts=0, norm=True, residual=True)
        elif kind == "zipf":
            _cache[kind] = synth.make_layer(0, wtype="nvfp4", bias="zipf")
    return _cache[kind]


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


@pytest.mark.parametrize("kind,T", [("norm", 8192), ("nvfp4", 8192), ("dense", 2048)])
def test_prefill_full_shape(kind, T):
    # Every token against the oracle (which runs on every host thread).
    # Residual layers are gated on the layer output with the residual add
    # off (one BF16 ulp of a residual stream with |x| >= 2 exceeds the
    # max-abs bar), and the add itself is checked exactly for every element:
    # one BF16 rounding of x + o.
    log(f"test: prefill full shape {kind} T={T}")
    L = full_layer(kind)
    dev = moe.DeviceLayer(L)
    x = synth.tokens(T, 2048, stream=900)
    out, idx, w = run(L, x, dev, residual=0)
    o = oracle.bf16_to_f64(out)
    assert np.all(np.isfinite(o))
    E = L["n_experts"]
    if E:
        check_routing_properties(L, idx, w)
    _, st = compare(dict(L, residual=0), x, out, idx if E else None, w if E else None,
                    what=f"prefill full {kind} T={T}")
    if L["residual"]:
        yr, idx_r, _ = run(L, x, dev, residual=1)
        assert np.array_equal(idx_r, idx)
        want = oracle.bf16_round_array(oracle.bf16_to_f64(x) + o)
        assert np.array_equal(yr, want)
    if E:
        counts = np.bincount(idx.reshape(-1), minlength=E)
        st["rows_per_expert_min_max"] = (int(counts.min()), int(counts.max()))
    log(f"  {st}")


@pytest.mark.parametrize("T", [9, 16, 32, 64, 128, 256])
def test_mid_batch_full_shape(T):
    # Between the decode path (up to 8 tokens) and the 8192-token prefill:
    # the full NVFP4 layer with the Zipf-biased router (the skew of the
    # batch-8 decode workload) through moe_prefill_layer, every token
    # against the oracle.
    log(f"test: mid batch full shape T={T}")
    L = full_layer("zipf")
    dev = moe.DeviceLayer(L)
    x = synth.tokens(T, 2048, stream=950 + T)
    out, idx, w = run(L, x, dev)
    check_routing_properties(L, idx, w)
    _, st = compare(L, x, out, idx, w, what=f"mid batch T={T}")
    st["distinct"] = len(np.unique(idx))
    log(f"  {st}")

"""GPU parity of the attention beside the MoE blocks (moe_attn_prep: per-head
Q/K RMSNorm, RoPE and the KV-cache write; moe_attn_decode: decode attention
with learned sinks and a sliding window) against the CPU oracle, through the
C ABI.

Inputs (seeded, synthetic): the fused QKV projection's output for each token
BF16(N(0, 1)) (a 2048-wide N(0, 1) activation times N(0, 0.02) weights has
about unit variance), per-head gains BF16(1 + 0.02 N(0, 1)), the cache
history BF16(N(0, 1)) keys and values, sinks N(0, 1) in FP32.  Shapes: GQA
32/4 heads of 128 (the pages' model), plus other group sizes; 513-position
windows in a ring of 544 slots; full-context layers up to 100,001 positions.

Bar: q and the written key rows equal the oracle's bits except for at most
1 in 10^4 elements one BF16 ulp apart (both sides round the same FP64
value; only summation order and FP64 math-library ulps differ); value rows
are copied bit-exact; the attention output meets the layer's output bar
(rel-L2 <= 2e-3, max-abs <= 1e-2 with the one-ulp allowance)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import check_outputs, from_dev_bits, log, to_dev_bits, wait_status

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a16_routed_expert_sigmoid_amd as moe  # noqa: E402

D = 128
BAD = 8  # status bit: a token's position was out of range


def bf16_ulp_diff(a, b):
    """|a - b| in BF16 ulps of b, elementwise (bits in, normal range)."""
    fa, fb = oracle.bf16_to_f64(a), oracle.bf16_to_f64(b)
    m, e = np.frexp(np.abs(fb))
    ulp = np.ldexp(1.0, e - 8)
    ulp[fb == 0] = 2.0 ** -133
    return np.abs(fa - fb) / ulp


# The cache's tile layout (the C header's formulas): element d of the slot
# at offset o of a 32-slot tile.
_O, _D = np.meshgrid(np.arange(32), np.arange(D), indexing="ij")
K_INDEX = (((_O // 4) % 2 * 4 + _D // 32) * 64 + (_D // 8) % 4 * 16 + (_O // 8) * 4 + _O % 4) * 8 + _D % 8
V_INDEX = ((_D // 16) * 64 + (_O // 8) * 16 + _D % 16) * 8 + _O % 8


def pack_cache(logical, index):
    """[B][slots][n_kv][D] -> [B][n_kv][slots/32][4096] in the tile layout."""
    B, slots, nkv, _ = logical.shape
    t = logical.reshape(B, slots // 32, 32, nkv, D).transpose(0, 3, 1, 2, 4)   # B, nkv, tiles, o, d
    out = np.empty((B, nkv, slots // 32, 32 * D), logical.dtype)
    out[..., index.ravel()] = t.reshape(B, nkv, slots // 32, 32 * D)
    return out


def unpack_cache(packed, index, slots):
    B, nkv = packed.shape[:2]
    t = packed.reshape(B, nkv, slots // 32, 32 * D)[..., index.ravel()].reshape(B, nkv, slots // 32, 32, D)
    return t.transpose(0, 2, 3, 1, 4).reshape(B, slots, nkv, D)


def check_rounded(gpu, ref, what):
    d = bf16_ulp_diff(gpu, ref)
    n = int(np.count_nonzero(d > 0))
    assert np.all(d <= 1.0), f"{what}: {np.max(d):.1f} ulp at {np.argwhere(d > 1)[:4]}"
    assert n <= max(1, 1e-4 * d.size), f"{what}: {n} of {d.size} elements one ulp apart"
    if n:
        log(f"  {what}: {n} of {d.size} elements one BF16 ulp from the oracle")


class Case:
    """One attention layer call: inputs, the oracle's results, the GPU's."""

    def __init__(self, n_q=32, n_kv=4, window=513, rope=1, slots=544, pos=(600,), seed=1, sinks=True,
                 theta=10000.0, eps=1e-6, max_ctx=0):
        self.B = B = len(pos)
        self.pos = np.array(pos, np.int64)
        self.a = dict(n_q=n_q, n_kv=n_kv, head_dim=D, window=window, rope=rope, rope_theta=theta,
                      eps=float(np.float32(eps)))
        self.desc = moe.moe_attn_desc(n_q, n_kv, D, window, rope, slots, theta, eps)
        self.n_q, self.n_kv, self.slots, self.window, self.max_ctx = n_q, n_kv, slots, window, max_ctx
        units = n_q + 2 * n_kv
        self.qkv = synth.normal_bf16(seed, 31, 0, 1.0, B * units * D).reshape(B, units * D)
        self.qg = synth.gain(D, 1000 + seed)
        self.kg = synth.gain(D, 2000 + seed)
        # history in the oracle's layout [B][slots][n_kv][D]
        self.kc = synth.normal_bf16(seed, 32, 0, 1.0, B * slots * n_kv * D).reshape(B, slots, n_kv, D)
        self.vc = synth.normal_bf16(seed, 33, 0, 1.0, B * slots * n_kv * D).reshape(B, slots, n_kv, D)
        self.sinks = synth.normal_f64(seed, 34, 0, 1.0, n_q).astype(np.float32) if sinks else None

    def valid(self, p):
        return p >= 0 and (self.window > 0 or p < self.slots)

    def span_ok(self, p):
        bound = self.max_ctx or (self.window or self.slots)
        lo = max(0, p - self.window + 1) if self.window else 0
        return self.valid(p) and p - lo + 1 <= bound

    def run_oracle(self):
        q, k, v = oracle.attn_prep(self.a, self.qkv, np.maximum(self.pos, 0), self.qg, self.kg)
        kc, vc = self.kc.copy(), self.vc.copy()
        for t, p in enumerate(self.pos):
            if self.valid(p):
                kc[t, p % self.slots] = k[t]
                vc[t, p % self.slots] = v[t]
        self.ref_q, self.ref_kc, self.ref_vc = q, kc, vc
        ok = [t for t in range(self.B) if self.span_ok(self.pos[t])]
        out = np.zeros((self.B, self.n_q, D), np.uint16)
        if ok:
            out[ok] = oracle.attn_decode(self.a, q[ok], kc[ok], vc[ok], self.pos[ok], self.sinks)
        self.ref_out = out
        return self

    def upload(self):
        self.d_qkv = to_dev_bits(self.qkv)
        self.d_pos = torch.from_numpy(self.pos).cuda()
        self.d_qg, self.d_kg = to_dev_bits(self.qg), to_dev_bits(self.kg)
        self.d_q = torch.empty((self.B, self.n_q, D), dtype=torch.int16, device="cuda")
        self.d_k = to_dev_bits(pack_cache(self.kc, K_INDEX))
        self.d_v = to_dev_bits(pack_cache(self.vc, V_INDEX))
        self.d_sinks = None if self.sinks is None else torch.from_numpy(self.sinks).cuda()
        self.d_out = torch.empty((self.B, self.n_q, D), dtype=torch.int16, device="cuda")
        self.ws_bytes = moe.moe_attn_workspace_bytes(self.desc, self.B, self.max_ctx)
        assert self.ws_bytes > 0
        self.d_ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        return self

    def launch(self):
        moe.moe_attn_prep(self.desc, self.d_qkv, self.d_pos, self.B, self.d_qg, self.d_kg, self.d_q, self.d_k,
                          self.d_v)
        moe.moe_attn_decode(self.desc, self.d_q, self.d_k, self.d_v, self.d_pos, self.B, self.d_out, self.d_ws,
                            self.ws_bytes, max_ctx=self.max_ctx, sinks=self.d_sinks)

    def launch_fused(self):
        moe.moe_attn_layer(self.desc, self.d_qkv, self.d_pos, self.B, self.d_qg, self.d_kg, self.d_k, self.d_v,
                           self.d_out, self.d_ws, self.ws_bytes, max_ctx=self.max_ctx, sinks=self.d_sinks)

    def fetch(self):
        torch.cuda.synchronize()
        self.g_q = from_dev_bits(self.d_q)
        self.g_out = from_dev_bits(self.d_out)
        self.status = wait_status(self.d_ws)
        return self

    def check(self, what, caches=True, q=True):
        ok = [t for t in range(self.B) if self.valid(self.pos[t])]
        bad = [t for t in range(self.B) if not self.valid(self.pos[t])]
        if ok and q:
            check_rounded(self.g_q[ok], self.ref_q[ok], f"{what} q")
        if q:
            assert np.all(self.g_q[bad] == 0), f"{what}: q of a bad position"
        if caches:
            gk = unpack_cache(from_dev_bits(self.d_k), K_INDEX, self.slots)
            gv = unpack_cache(from_dev_bits(self.d_v), V_INDEX, self.slots)
            assert np.array_equal(gv, self.ref_vc), f"{what}: value cache"
            check_rounded(gk, self.ref_kc, f"{what} key cache")
        good = [t for t in range(self.B) if self.span_ok(self.pos[t])]
        out_bad = [t for t in range(self.B) if t not in good]
        assert np.all(self.g_out[out_bad] == 0), f"{what}: output of a bad position"
        if good:
            st = check_outputs(self.g_out[good].reshape(len(good), -1), self.ref_out[good].reshape(len(good), -1),
                               what)
            log(f"  {what}: rel-L2 {st['rel_l2']:.2e} max-abs {st['max_abs']:.2e} bit-exact {st['bit_exact']:.4f}")
        want = 0 if not out_bad else BAD
        assert self.status == want, f"{what}: status {self.status}"


def run(what, **kw):
    log(f"test: {what} {kw}")
    c = Case(**kw)
    c.upload()
    c.launch()
    c.fetch()
    c.run_oracle()
    c.check(what)
    return c


@pytest.mark.parametrize("kw", [
    dict(window=0, rope=0, slots=64, pos=(0, 31, 63)),                      # full context, one chunk
    dict(window=17, rope=1, slots=32, pos=(5, 40, 1000)),                   # window in a small ring
    dict(window=513, rope=1, slots=544, pos=(0, 512, 543, 100000)),         # the model's window layers
    dict(window=513, rope=1, slots=544, pos=(777,), sinks=False),
    dict(window=0, rope=0, slots=2048, pos=(2047, 700), n_q=64, n_kv=4),    # 16 heads a group, split
    dict(window=0, rope=1, slots=1024, pos=(1023, 0), n_q=4, n_kv=4),       # one head a group
    dict(window=100, rope=1, slots=128, pos=(99, 100, 1234, 5, 127), n_q=16, n_kv=8),
    dict(window=0, rope=0, slots=8192, pos=(8191, 40, 3000)),               # chunks per token differ
    dict(window=2000, rope=1, slots=2016, pos=(5000, 1999, 2000)),          # split window over a ring
    dict(window=0, rope=1, slots=4096, pos=(4000,), theta=1e6, eps=1e-5),
])
def test_attn_matches_oracle(kw):
    run("attn", **kw)


FUSED_CASES = [
    dict(window=513, rope=1, slots=544, pos=(0, 512, 543, 100000)),
    dict(window=0, rope=0, slots=2048, pos=(2047, 700), n_q=64, n_kv=4),
    dict(window=0, rope=0, slots=8192, pos=(8191, 40, 3000)),
    dict(window=2000, rope=1, slots=2016, pos=(5000, 1999, 2000)),
    dict(window=17, rope=1, slots=32, pos=(5, 40, 1000)),
    dict(window=0, rope=1, slots=1024, pos=(1023, 0), n_q=4, n_kv=4),
    dict(window=0, rope=0, slots=64, pos=(-1, 5, 64, 63)),
    dict(window=0, rope=0, slots=4096, pos=(3000, 100), max_ctx=2000),
    dict(window=0, rope=0, slots=100032, pos=(100000,), seed=5),
]


@pytest.mark.parametrize("kw", FUSED_CASES)
def test_attn_layer_fused_equals_prep_then_decode(kw):
    # the fused call gives the two calls' outputs and cache contents bit for
    # bit, and meets the oracle bar on its own
    log(f"test: fused attention layer {kw}")
    c1 = Case(**kw).upload()
    c1.launch()
    c1.fetch()
    c2 = Case(**kw).upload()
    c2.launch_fused()
    c2.fetch()
    assert np.array_equal(c2.g_out, c1.g_out)
    assert torch.equal(c2.d_k, c1.d_k) and torch.equal(c2.d_v, c1.d_v)
    assert c2.status == c1.status
    c2.run_oracle().check("fused attention layer", q=False)


def test_attn_layer_fused_graph_replays():
    c = Case(window=513, rope=1, slots=544, pos=(1000, 20), seed=12).upload()
    k0, v0 = c.d_k.clone(), c.d_v.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.launch_fused()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c.launch_fused()
    for pos in ((1000, 20), (5000, 512), (3, 100000)):
        c.pos = np.array(pos, np.int64)
        c.d_pos.copy_(torch.from_numpy(c.pos))
        c.d_k.copy_(k0)
        c.d_v.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        c.fetch()
        c.run_oracle().check(f"fused graph replay {pos}", q=False)


def test_attn_full_context_100k_one_token():
    # the pages' decode measurement: batch 1 at 100K context (full layers)
    run("attn 100K", window=0, rope=0, slots=100032, pos=(100000,), seed=5)


def test_attn_full_context_batch4_long():
    run("attn long B=4", window=0, rope=0, slots=65536, pos=(65535, 30000, 777, 65000), seed=6)


def test_attn_window_batch8():
    run("attn window B=8", window=513, rope=1, slots=544,
        pos=(0, 1, 511, 512, 513, 4096, 99999, 262143), seed=7)


def test_attn_bad_positions_give_zeros_and_status():
    c = run("attn bad positions", window=0, rope=0, slots=64, pos=(-1, 5, 64, 63), seed=8)
    # the caches of the bad tokens are untouched
    gk = unpack_cache(from_dev_bits(c.d_k), K_INDEX, c.slots)
    assert np.array_equal(gk[[0, 2]], c.kc[[0, 2]])


def test_attn_max_ctx_bound():
    # token 0 attends 3001 positions, more than max_ctx = 2000
    run("attn max_ctx short", window=0, rope=0, slots=4096, pos=(3000, 100), max_ctx=2000, seed=9)
    run("attn max_ctx enough", window=0, rope=0, slots=4096, pos=(3000, 100), max_ctx=3001, seed=9)


def test_attn_repeat_is_deterministic():
    c = Case(window=0, rope=0, slots=8192, pos=(8000, 5000), seed=10).upload()
    k0, v0 = c.d_k.clone(), c.d_v.clone()
    c.launch()
    first = c.fetch().g_out.copy()
    c.d_k.copy_(k0)
    c.d_v.copy_(v0)
    c.launch()
    assert np.array_equal(c.fetch().g_out, first)


def test_attn_graph_replays_follow_device_positions():
    # prep + decode captured once; each replay reads the positions from
    # device memory, which the host changes between replays.
    c = Case(window=513, rope=1, slots=544, pos=(1000, 20), seed=11).upload()
    k0, v0 = c.d_k.clone(), c.d_v.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.launch()  # warm-up outside the graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c.launch()
    for pos in ((1000, 20), (5000, 512), (3, 100000)):
        c.pos = np.array(pos, np.int64)
        c.d_pos.copy_(torch.from_numpy(c.pos))
        c.d_k.copy_(k0)
        c.d_v.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        c.fetch()
        replay = c.g_out.copy()
        c.run_oracle().check(f"graph replay {pos}")
        c.d_k.copy_(k0)
        c.d_v.copy_(v0)
        c.launch()
        assert np.array_equal(c.fetch().g_out, replay), pos


def test_pack_helpers_round_trip():
    x = np.arange(2 * 64 * 4 * D, dtype=np.uint16).reshape(2, 64, 4, D)
    for idx in (K_INDEX, V_INDEX):
        assert np.array_equal(unpack_cache(pack_cache(x, idx), idx, 64), x)


@pytest.mark.parametrize("window,slots,first,n", [(0, 256, 0, 256), (513, 544, 1000, 600), (0, 64, 50, 20)])
def test_kv_write_places_rows_in_the_layout(window, slots, first, n):
    # rows of positions first .. first + n - 1 (later positions of a ring
    # overwrite earlier ones in the same slot: written here one call each,
    # in position order); positions beyond a full layer's slots are skipped
    log(f"test: kv_write window={window} slots={slots} first={first} n={n}")
    B, nkv = 2, 4
    desc = moe.moe_attn_desc(32, nkv, D, window, 0, slots, 0.0, 1e-6)
    k = synth.normal_bf16(77, 1, 0, 1.0, B * n * nkv * D).reshape(B, n, nkv, D)
    v = synth.normal_bf16(77, 2, 0, 1.0, B * n * nkv * D).reshape(B, n, nkv, D)
    kc0 = synth.normal_bf16(77, 3, 0, 1.0, B * slots * nkv * D).reshape(B, slots, nkv, D)
    d_k, d_v = to_dev_bits(pack_cache(kc0, K_INDEX)), to_dev_bits(pack_cache(kc0, V_INDEX))
    ref_k, ref_v = kc0.copy(), kc0.copy()
    for i in range(n):
        p = first + i
        if window == 0 and p >= slots:
            continue
        ref_k[:, p % slots] = k[:, i]
        ref_v[:, p % slots] = v[:, i]
    # one position per call keeps the ring's overwrite order
    step = n if window == 0 or n <= slots else 1
    for i0 in range(0, n, step):
        m = min(step, n - i0)
        pos = torch.from_numpy(np.array([[first + i0 + i for i in range(m)]] * B, np.int64)).cuda()
        moe.moe_attn_kv_write(desc, to_dev_bits(k[:, i0:i0 + m]), to_dev_bits(v[:, i0:i0 + m]), pos, m, B, d_k, d_v)
    torch.cuda.synchronize()
    assert np.array_equal(unpack_cache(from_dev_bits(d_k), K_INDEX, slots), ref_k)
    assert np.array_equal(unpack_cache(from_dev_bits(d_v), V_INDEX, slots), ref_v)

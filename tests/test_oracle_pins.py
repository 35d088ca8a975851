"""Pins of the CPU oracle against facts fixed outside it.

Each test names what fixes the expected values: a format specification or
a library decoder, hand-worked rounding ties, a closed form, an invariant of
top-k selection, or a brute-force dense evaluation of every expert with a
gate vector (tests/bruteforce.py) that shares no code with the oracle.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def tiny_layer(layer_id=0, H=64, I=32, Is=32, E=8, k=2, wtype="nvfp4", **kw):
    return synth.make_layer(layer_id, hidden=H, inter=I, shared_inter=Is, n_experts=E, top_k=k,
                            wtype=wtype, **kw)


# ---------------------------------------------------------------- formats

def test_e2m1_matches_ocp_table():
    # OCP MX v1.0, FP4 E2M1 (golden/e2m1_ocp.txt)
    for code, val in _read_golden("e2m1_ocp.txt"):
        got = oracle.e2m1_value(int(code))
        assert got == float(val) and np.signbit(got) == np.signbit(float(val)), code


def test_e4m3_all_256_codes_match_torch_float8():
    # library decoder: torch.float8_e4m3fn (OCP E4M3FN)
    ref = bf.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        got = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c] and np.signbit(got) == np.signbit(ref[c]), c
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_bf16_round_hand_worked_ties():
    for v, bits in _read_golden("bf16_ties.txt"):
        assert oracle.bf16_round(float.fromhex(v)) == int(bits, 16), v
    assert oracle.bf16_round(float("nan")) & 0x7FFF > 0x7F80


def test_bf16_round_matches_torch_on_fp32_inputs():
    # For FP32-representable inputs torch's FP32->BF16 RNE is a single rounding.
    rng = np.random.default_rng(1)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(5000) * 1e-38).astype(np.float32),
                        (rng.standard_normal(5000) * 1e37).astype(np.float32)])
    # force exact ties: low 16 bits = 0x8000
    tie = (f.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = np.concatenate([f, tie.view(np.float32)])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_round(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_round_array_equals_scalar_rounding():
    v = np.concatenate([np.random.default_rng(4).standard_normal(3000) * 10.0 ** np.arange(-3, 3).repeat(500),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, np.inf, -np.inf, 1e39]])
    got = oracle.bf16_round_array(v)
    assert np.array_equal(got, np.array([oracle.bf16_round(x) for x in v], np.uint16))


def test_bf16_value_exact():
    for bits in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x4049):
        ref = bf.bf16_bits_to_f64(np.array([bits], np.uint16))[0]
        assert oracle.bf16_value(bits) == ref


def test_decode_nvfp4_byte_order_and_nan_count():
    # One row of two blocks.  Block 0: scale 0x38 (=1.0), nibble byte j =
    # code j | code (j+8) << 4, so element i must decode to E2M1[i].
    # Block 1: scale 0x7F (NaN) -> counted.
    blk0 = [0x38] + [j | ((j + 8) << 4) for j in range(8)]
    blk1 = [0x7F] + [0x21] * 8
    src = np.array(blk0 + blk1, dtype=np.uint8)
    vals, nan = oracle.decode_nvfp4(src, 1, 32, 0.5)
    assert nan == 1
    assert np.array_equal(vals[0, :16], bf.E2M1 * 0.5)
    assert np.all(np.isnan(vals[0, 16:]))


def test_decode_nvfp4_matches_bruteforce_decoder():
    m, s = synth.nvfp4_stack(5, 0, 1, 1, 64, 128)
    ref = bf.decode_matrix(m[0], 64, 128, "nvfp4", float(s[0]))
    got, nan = oracle.decode_nvfp4(m[0], 64, 128, float(s[0]))
    assert nan == 0 and np.array_equal(got, ref)


def test_fp4_round_trip_every_e2m1_x_e4m3_code():
    # decode(encode(v)) == v for every representable v = E2M1[q] * E4M3[s]
    # (tensor scale 1): row 0 pins the tensor scale to exactly 1 through
    # amax = 6 * 448; row (s, q) holds 6*E4M3[s] (so the block scale must
    # be s) and the value E2M1[q]*E4M3[s].
    scales = list(range(1, 0x7F))
    rows = [np.r_[6.0 * 448.0, np.zeros(15)]]
    expect = [rows[0]]
    for sc in scales:
        sv = oracle.e4m3_value(sc)
        for q in range(16):
            r = np.zeros(16)
            r[0] = 6.0 * sv
            r[1] = bf.E2M1[q] * sv
            rows.append(r)
            expect.append(r)
    W = np.stack(rows)
    gg, S = synth.quantize_nvfp4(W)
    assert S == 1.0
    got, nan = oracle.decode_nvfp4(gg, W.shape[0], 16, S)
    assert nan == 0
    assert np.array_equal(got, np.stack(expect))
    assert np.array_equal(gg[1:, 0], np.repeat(np.array(scales, np.uint8), 16))


# ---------------------------------------------------------------- closed forms

def test_zero_input_full_tie():
    # x = 0, b = 0: every logit 0, every score 0.5 -> a full tie; lower index
    # first gives experts 0..k-1, each weight 1/k, output exactly 0, flagged.
    L = tiny_layer(k=3)
    r = oracle.moe_tokens(L, np.zeros((1, 64), np.uint16))
    assert list(r["idx"][0]) == [0, 1, 2]
    assert np.allclose(r["w"][0], 1.0 / 3.0, rtol=0, atol=1e-15)
    assert r["flag"][0] == 1
    assert np.all(r["out"] == 0)


def _constant_matrix(rows, cols, code, scale_code):
    blk = np.array([scale_code] + [code | (code << 4)] * 8, dtype=np.uint8)
    return np.tile(blk, (rows, cols // 16)).reshape(rows, cols // 16 * 9)


def test_constant_code_weights_closed_form():
    # Every gate element = E2M1[cg]*E4M3[sg]*Sg etc., so every g_n equals
    # BF16(a_g * sum(x)), every u_n = BF16(a_u * sum(x)), every h_n the same,
    # and y_m = BF16(a_d * I * h) for every expert; with identical experts
    # the renormalised weights sum to 1, so o = BF16(y + y_shared).
    H, I, Is, E, k = 64, 32, 48, 4, 2
    L = tiny_layer(H=H, I=I, Is=Is, E=E, k=k)
    cg, cu, cd, sg, su, sd = 3, 10, 5, 0x30, 0x38, 0x2C  # codes 1.5, -1, 3; scales 0.5, 1, 0.375
    Sg, Su, Sd = 0.25, 2.0, 0.125
    L["w_gate"] = np.stack([_constant_matrix(I, H, cg, sg)] * E)
    L["w_up"] = np.stack([_constant_matrix(I, H, cu, su)] * E)
    L["w_down"] = np.stack([_constant_matrix(H, I, cd, sd)] * E)
    L["w_scale"] = np.tile(np.array([Sg, Su, Sd], np.float32), (E, 1))
    L["sh_gate"] = _constant_matrix(Is, H, cg, sg)
    L["sh_up"] = _constant_matrix(Is, H, cu, su)
    L["sh_down"] = _constant_matrix(H, Is, cd, sd)
    L["sh_scale"] = np.array([Sg, Su, Sd], np.float32)
    x = synth.tokens(1, H, stream=3, sigma=0.05)
    xs = float(np.sum(bf.bf16_bits_to_f64(x[0])))
    e4 = bf.e4m3_decode(np.array([sg, su, sd], np.uint8))
    ag = bf.E2M1[cg] * e4[0] * Sg
    au = bf.E2M1[cu] * e4[1] * Su
    ad = bf.E2M1[cd] * e4[2] * Sd
    g = bf.bf16(ag * xs)
    u = bf.bf16(au * xs)
    h = bf.bf16(g / (1 + np.exp(-g)) * u)
    y = bf.bf16(ad * I * h)
    ysh = bf.bf16(ad * Is * h)
    expect = bf.bf16_bits(y + ysh)
    r = oracle.moe_tokens(L, x)
    assert np.all(r["out"][0] == expect)


@pytest.mark.parametrize("c", [0.3125, 2.0 ** -10])
def test_rmsnorm_constant_input_closed_form(c):
    # x_k = c for all k: mean(x^2) = c^2, xn_k = BF16(c / sqrt(c^2 + eps) * g_k).
    # A one-expert, no-shared layer with identity-like probing is awkward, so
    # probe xn through the router: with Wr = e_j (one-hot rows, BF16 1.0),
    # logit_e = xn_{j(e)} exactly.  At c = 2^-10, c^2 is close to eps = 1e-6,
    # so the eps term visibly moves xn.
    H, E = 64, 8
    L = tiny_layer(H=H, E=E, k=1, norm=True)
    x = np.full((1, H), bf.bf16_bits(np.array([c]))[0], np.uint16)
    Wr = np.zeros((E, H), np.uint16)
    for e in range(E):
        Wr[e, 5 * e] = 0x3F80
    L["router_w"] = Wr
    L["router_b"] = np.zeros(E, np.float32)
    r = oracle.moe_tokens(L, x)
    g = bf.bf16_bits_to_f64(L["norm_gain"])
    xn = bf.bf16(c / np.sqrt(c * c + L["eps"]) * g)
    assert np.array_equal(r["logits"][0], xn[5 * np.arange(E)])


# ---------------------------------------------------------------- routing invariants

@pytest.mark.parametrize("bias", ["zero", "zipf"])
def test_topk_invariants(bias):
    L = tiny_layer(H=128, I=32, Is=32, E=64, k=6, bias=bias if bias == "zero" else "none")
    if bias == "zipf":
        L["router_b"] = synth.zipf_offset(64)
    x = synth.tokens(16, 128, stream=11)
    r = oracle.moe_tokens(L, x)
    for t in range(16):
        idx, w, lg = r["idx"][t], r["w"][t], r["logits"][t]
        assert len(set(idx)) == 6 and idx.min() >= 0 and idx.max() < 64
        others = np.setdiff1d(np.arange(64), idx)
        assert lg[idx].min() >= lg[others].max()
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(np.diff(w) <= 0)
        assert np.all(np.diff(lg[idx]) <= 0)
        s = 1 / (1 + np.exp(-lg))
        assert np.allclose(w, s[idx] / s[idx].sum(), rtol=1e-14, atol=0)


def test_forced_bias_selects_chosen_set():
    L = tiny_layer(H=128, E=64, k=6)
    chosen = [3, 17, 22, 40, 41, 63]
    b = np.zeros(64, np.float32)
    b[chosen] = 30.0
    L["router_b"] = b
    r = oracle.moe_tokens(L, synth.tokens(4, 128, stream=5))
    for t in range(4):
        assert sorted(r["idx"][t]) == chosen


def test_permutation_equivariance():
    # Relabelling experts permutes the selected indices and leaves the output
    # bit-identical.
    L = tiny_layer(H=128, I=32, Is=32, E=16, k=4, bias="zipf")
    x = synth.tokens(6, 128, stream=9)
    perm = np.random.default_rng(3).permutation(16)  # new expert p <- old expert perm[p]
    P = dict(L)
    for key in ("router_w", "router_b", "w_gate", "w_up", "w_down", "w_scale"):
        P[key] = np.ascontiguousarray(L[key][perm])
    r0 = oracle.moe_tokens(L, x)
    r1 = oracle.moe_tokens(P, x)
    inv = np.argsort(perm)
    assert np.array_equal(r0["out"], r1["out"])
    assert np.array_equal(inv[r0["idx"]], r1["idx"])
    assert np.array_equal(r0["w"], r1["w"])


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("wtype", ["nvfp4", "bf16"])
def test_one_hot_gate_matches_dense_bruteforce(wtype):
    # k = 1 with a +30 bias on one expert: w = 1 exactly, so the layer is
    # BF16(FFN_e*(x) + FFN_shared(x)) -- checked against evaluating every
    # expert densely and mixing with a one-hot gate.
    for target in (0, 5):
        L = tiny_layer(E=8, k=1, wtype=wtype)
        b = np.zeros(8, np.float32)
        b[target] = 30.0
        L["router_b"] = b
        x = synth.tokens(3, 64, stream=target)
        r = oracle.moe_tokens(L, x)
        ref, sets = bf.dense_moe(L, x)
        assert all(s == {target} for s in sets)
        assert np.all(r["idx"] == target) and np.all(r["w"] == 1.0)
        assert np.array_equal(r["out"], ref)


@pytest.mark.parametrize("cfg", [
    dict(wtype="nvfp4", k=6, bias="zero"),
    dict(wtype="nvfp4", k=6, bias="zipf", norm=True, residual=True),
    dict(wtype="bf16", k=3, bias="zero"),
])
def test_topk_matches_dense_bruteforce(cfg):
    wtype, k = cfg["wtype"], cfg["k"]
    L = synth.make_layer(7, hidden=128, inter=64, shared_inter=96, n_experts=32, top_k=k, wtype=wtype,
                         bias="zero" if cfg["bias"] == "zero" else "none",
                         norm=cfg.get("norm", False), residual=cfg.get("residual", False))
    if cfg["bias"] == "zipf":
        L["router_b"] = synth.zipf_offset(32)
    x = synth.tokens(8, 128, stream=21)
    r = oracle.moe_tokens(L, x)
    ref, sets = bf.dense_moe(L, x)
    for t in range(8):
        if r["flag"][t]:
            continue
        assert set(r["idx"][t]) == sets[t]
    # Summation order differs (selected-order vs dense gate @ Y), so allow the
    # rare FP64 last-bit effect on a BF16 tie; in practice all bits agree.
    o = bf.bf16_bits_to_f64(r["out"])
    e = bf.bf16_bits_to_f64(ref)
    assert np.mean(r["out"] == ref) > 0.999
    assert np.max(np.abs(o - e) / np.maximum(np.abs(e), 1e-30)) <= 2.0 ** -7


def test_dense_layer_is_shared_expert_alone():
    # n_experts = 0: the layer is one SwiGLU of width shared_inter.
    L = synth.make_layer(3, hidden=128, inter=0, shared_inter=160, n_experts=0, wtype="nvfp4")
    x = synth.tokens(2, 128, stream=2)
    r = oracle.moe_tokens(L, x)
    ref, _ = bf.dense_moe(L, x)
    assert np.array_equal(r["out"], ref)


def test_nvfp4_equals_bf16_at_power_of_two_tensor_scales():
    # With power-of-two tensor scales every NVFP4 weight (<= 6 significant
    # bits) is exactly a BF16 number, so the NVFP4 layer and the BF16 layer
    # holding the decoded weights must agree bit for bit.
    H, I, Is, E = 128, 64, 64, 16
    L4 = synth.make_layer(2, hidden=H, inter=I, shared_inter=Is, n_experts=E, top_k=4,
                          wtype="nvfp4", pow2_tensor_scale=True, bias="zipf")
    assert all(np.log2(s) == np.round(np.log2(s)) for s in L4["w_scale"].ravel())

    def to_bf16(m, rows, cols, s):
        v, nan = oracle.decode_nvfp4(m, rows, cols, float(s))
        assert nan == 0
        f = v.astype(np.float32)
        assert np.array_equal(f.astype(np.float64), v)
        bits = f.view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)
        return (bits >> 16).astype(np.uint16)

    LB = dict(L4, wtype="bf16", w_scale=None, sh_scale=None)
    LB["w_gate"] = np.stack([to_bf16(L4["w_gate"][e], I, H, L4["w_scale"][e, 0]) for e in range(E)])
    LB["w_up"] = np.stack([to_bf16(L4["w_up"][e], I, H, L4["w_scale"][e, 1]) for e in range(E)])
    LB["w_down"] = np.stack([to_bf16(L4["w_down"][e], H, I, L4["w_scale"][e, 2]) for e in range(E)])
    LB["sh_gate"] = to_bf16(L4["sh_gate"], Is, H, L4["sh_scale"][0])
    LB["sh_up"] = to_bf16(L4["sh_up"], Is, H, L4["sh_scale"][1])
    LB["sh_down"] = to_bf16(L4["sh_down"], H, Is, L4["sh_scale"][2])
    x = synth.tokens(4, H, stream=4)
    a = oracle.moe_tokens(L4, x)
    b = oracle.moe_tokens(LB, x)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["idx"], b["idx"])


def test_batch_equals_independent_tokens():
    # Tokens do not interact (decode batch, prefill): T tokens at once equal T
    # single-token calls.
    L = tiny_layer(H=128, E=16, k=4, bias="zipf")
    x = synth.tokens(5, 128, stream=8)
    r = oracle.moe_tokens(L, x)
    for t in range(5):
        r1 = oracle.moe_tokens(L, x[t:t + 1])
        assert np.array_equal(r1["out"][0], r["out"][t]) and np.array_equal(r1["idx"][0], r["idx"][t])


def test_nan_scale_reported():
    L = tiny_layer(E=4, k=4)
    L["sh_gate"] = L["sh_gate"].copy()
    L["sh_gate"][0, 0] = 0x7F
    r = oracle.moe_tokens(L, synth.tokens(1, 64))
    assert r["nan_tokens"] == 1


def test_full_shape_one_hot_matches_dense_bruteforce():
    # Full width (H 2048, I 512) on a few experts: the one-hot case at the
    # real matrix sizes.
    L = synth.make_layer(1, hidden=2048, inter=512, shared_inter=512, n_experts=4, top_k=1)
    b = np.zeros(4, np.float32)
    b[2] = 30.0
    L["router_b"] = b
    x = synth.tokens(1, 2048, stream=1)
    r = oracle.moe_tokens(L, x)
    ref, _ = bf.dense_moe(L, x)
    assert np.array_equal(r["out"], ref)


# ---------------------------------------------------------------- near-tie flag
#
# The flag marks a token whose k-th and (k+1)-th sigmoid scores differ by
# less than 1e-5 (then more than one expert set is a correct selection).
# With x = 0 every router dot product is exactly 0, so each logit equals its
# FP32 bias and the cases below are set by hand.  Near 0 the sigmoid has
# slope 1/4 and no curvature, so a logit gap d gives a score gap of d/4 to
# within 1e-13: d = 3.6e-5 -> 9.0e-6 (flagged), d = 4.4e-5 -> 1.1e-5 (not).
# Each case fails one plausible mistake: always 1, always 0, the gap taken
# one rank too high or too low, or the gap taken on the logits.

def _flag_of(biases, k):
    L = tiny_layer(E=len(biases), k=k)
    L["router_b"] = np.asarray(biases, np.float32)
    r = oracle.moe_tokens(L, np.zeros((1, 64), np.uint16))
    return int(r["flag"][0]), r


def test_flag_gap_just_below_threshold():
    # ranks: 5, 5 (experts 1, 4), then 0 (expert 3) = k-th, then -3.6e-5
    # (expert 5) = (k+1)-th: score gap 9.0e-6 < 1e-5 -> flagged.  A flag
    # on the logits (gap 3.6e-5) would not fire.
    f, r = _flag_of([-5, 5, -5, 0, 5, -3.6e-5, -5, -5], 3)
    assert f == 1
    assert set(r["idx"][0]) == {1, 3, 4}


def test_flag_gap_just_above_threshold():
    f, r = _flag_of([-5, 5, -5, 0, 5, -4.4e-5, -5, -5], 3)
    assert f == 0
    assert set(r["idx"][0]) == {1, 3, 4}


def test_flag_near_tie_one_rank_above_boundary_is_not_flagged():
    # ranks 2 and 3 (0.5 and 0.5 - 2e-6, score gap ~4.7e-7) nearly tie, but
    # the k-th (k = 3: 0.5 - 2e-6) and (k+1)-th (-2) are far apart.
    f, r = _flag_of([3, 0.5, -5, 0.5 - 2e-6, -2, -5, -5, -5], 3)
    assert f == 0
    assert set(r["idx"][0]) == {0, 1, 3}


def test_flag_near_tie_one_rank_below_boundary_is_not_flagged():
    # ranks 4 and 5 (-1 and -1 - 1e-6) nearly tie; the boundary gap
    # sigmoid(1) - sigmoid(-1) is 0.46.
    f, r = _flag_of([3, 2, -5, 1, -1, -1 - 1e-6, -5, -5], 3)
    assert f == 0
    assert set(r["idx"][0]) == {0, 1, 3}


@pytest.mark.parametrize("base", [28.0, -22.0])
def test_flag_saturated_scores_tie_while_logits_differ(base):
    # Logits one apart deep in either tail: sigmoid(28) - sigmoid(27) is
    # about 1.2e-12 and sigmoid(-22) - sigmoid(-23) about 1.8e-10, both far
    # below 1e-5, while the logit gap is 1.  Selection still follows the
    # logits exactly: experts 6, 2, 7 (descending).
    b = np.full(8, base - 10.0)
    b[[6, 2, 7, 0]] = [base + 2, base + 1, base, base - 1]
    f, r = _flag_of(b, 3)
    assert f == 1
    assert list(r["idx"][0]) == [6, 2, 7]


def test_flag_all_experts_selected_is_never_flagged():
    # k = E: every expert is selected, so no other set exists.
    f, r = _flag_of([0.0] * 8, 8)
    assert f == 0
    assert list(r["idx"][0]) == list(range(8))


def test_threaded_oracle_is_bit_identical():
    # Tokens are independent and each is owned by one thread.
    L = tiny_layer(H=128, E=16, k=4, bias="zipf", norm=True, residual=True)
    x = synth.tokens(37, 128, stream=12)
    a = oracle.moe_tokens(L, x, threads=1)
    for n in (2, 5, 64):
        b = oracle.moe_tokens(L, x, threads=n)
        for key in ("out", "idx", "w", "flag", "logits"):
            assert np.array_equal(a[key], b[key]), (n, key)


# ---------------------------------------------------------------- dense NVFP4 GEMV

def test_gemv_constant_code_closed_form():
    # every element E2M1[c] * E4M3[s] * S: y_n = BF16(E2M1[c] E4M3[s] S sum(x))
    rows, cols, c, sc, S = 24, 96, 11, 0x3A, 0.75   # code 11 = -1.5, scale 0x3A = 1.25
    m = _constant_matrix(rows, cols, c, sc)
    x = synth.tokens(3, cols, stream=31)
    y, nan = oracle.gemv_nvfp4(m, rows, cols, S, x)
    assert nan == 0
    a = bf.E2M1[c] * bf.e4m3_decode(np.array([sc], np.uint8))[0] * S
    want = bf.bf16_bits(a * bf.bf16_bits_to_f64(x).sum(axis=1))
    assert np.array_equal(y, np.repeat(want[:, None], rows, axis=1))


def test_gemv_one_hot_input_reads_one_column():
    # x = e_j: y_n = BF16(W[n][j]); with a power-of-two tensor scale every
    # NVFP4 value is a BF16 number, so y is exactly column j of the decoded
    # matrix (a transposed operand or a wrong nibble order would not be).
    rows, cols = 40, 64
    m, s = synth.nvfp4_stack(9, 0, 1, 1, rows, cols, pow2_tensor_scale=True)
    W = bf.decode_matrix(m[0], rows, cols, "nvfp4", float(s[0]))
    for j in (0, 1, 8, 15, 17, 63):
        x = np.zeros((1, cols), np.uint16)
        x[0, j] = 0x3F80  # 1.0
        y, _ = oracle.gemv_nvfp4(m[0], rows, cols, float(s[0]), x)
        assert np.array_equal(bf.bf16_bits_to_f64(y[0]), W[:, j]), j


def test_gemv_matches_bruteforce_decode_and_matmul():
    rows, cols = 72, 320
    m, s = synth.nvfp4_stack(10, 0, 1, 1, rows, cols)
    x = synth.tokens(4, cols, stream=32)
    y, nan = oracle.gemv_nvfp4(m[0], rows, cols, float(s[0]), x)
    W = bf.decode_matrix(m[0], rows, cols, "nvfp4", float(s[0]))
    want = bf.bf16_bits(bf.bf16_bits_to_f64(x) @ W.T)
    assert nan == 0 and np.array_equal(y, want)


def test_gemv_counts_nan_scales():
    m = _constant_matrix(8, 32, 3, 0x38).copy()
    m[2, 9] = 0xFF  # scale byte of row 2, block 1
    _, nan = oracle.gemv_nvfp4(m, 8, 32, 1.0, synth.tokens(2, 32, stream=1))
    assert nan == 1

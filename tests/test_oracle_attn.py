"""Pins of the attention oracle (Q/K norm, RoPE, decode attention with
learned sinks and a sliding window) against facts fixed outside it.

Expected values come from closed forms worked by hand, from rotations
computed as complex multiplications in NumPy, and from torch's
scaled_dot_product_attention in float64, the library routine the decode
reduces to once GQA heads are repeated, the window is an additive -inf mask
and the sink is an extra key of logit ``sink`` and value zero.  BF16
rounding of expected values uses tests/bruteforce.py, which shares no code
with the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import bruteforce as bf

NQ, NKV, D = 32, 4, 128
G = NQ // NKV


def cfg(**kw):
    a = dict(n_q=NQ, n_kv=NKV, head_dim=D, window=0, rope=0, rope_theta=10000.0, eps=1e-6)
    a.update(kw)
    return a


def bits(v):
    return bf.bf16_bits(np.asarray(v, dtype=np.float64))


def val(b):
    return bf.bf16_bits_to_f64(b)


def rand_bits(seed, n, sigma=1.0):
    return synth.normal_bf16(seed, 7, 0, sigma, n)


def qkv_of(q_heads, k_heads, v_heads):
    """Concatenate head vectors (float values, BF16-exact) into one token."""
    return bits(np.concatenate([np.ravel(q_heads), np.ravel(k_heads), np.ravel(v_heads)]))[None, :]


# ------------------------------------------------------------ Q/K norm

def test_head_norm_constant_input_gives_the_gain():
    # x_d = c for every d: mean(x^2) = c^2, so x / rms = 1 and out = BF16(g).
    qg = rand_bits(1, D, 0.3)
    kg = rand_bits(2, D, 0.3)
    qkv = qkv_of(np.full((NQ, D), 2.0), np.full((NKV, D), -0.5), val(rand_bits(3, NKV * D)))
    q, k, _ = oracle.attn_prep(cfg(), qkv, [5], qg, kg)
    assert np.array_equal(q[0], np.tile(qg, (NQ, 1)))
    assert np.array_equal(k[0], np.tile(bits(-val(kg)), (NKV, 1)))


def test_head_norm_eps_inside_the_root():
    # c = 1, eps = 3: 1 / sqrt(1 + 3) = 0.5 exactly, so out = g / 2.
    qg = rand_bits(4, D, 0.3)
    qkv = qkv_of(np.ones((NQ, D)), np.ones((NKV, D)), np.zeros((NKV, D)))
    q, k, _ = oracle.attn_prep(cfg(eps=3.0), qkv, [0], qg, qg)
    assert np.array_equal(q[0], np.tile(bits(val(qg) / 2), (NQ, 1)))


def test_head_norm_is_per_head():
    # Scaling one head's input leaves every head's output unchanged; heads
    # normalised together would change.
    qg = bits(np.ones(D))
    x = val(rand_bits(5, (NQ + 2 * NKV) * D)).reshape(-1, D)
    q0, k0, _ = oracle.attn_prep(cfg(eps=0.0), bits(x.ravel())[None], [0], qg, qg)
    x[3] *= 64.0
    x[NQ + 1] *= 0.25
    q1, k1, _ = oracle.attn_prep(cfg(eps=0.0), bits(x.ravel())[None], [0], qg, qg)
    assert np.array_equal(q0, q1) and np.array_equal(k0, k1)


def test_v_heads_pass_through():
    qkv = rand_bits(6, (NQ + 2 * NKV) * D)[None]
    _, _, v = oracle.attn_prep(cfg(rope=1), qkv, [77], rand_bits(7, D), rand_bits(8, D))
    assert np.array_equal(v[0].ravel(), qkv[0, (NQ + NKV) * D:])


# ------------------------------------------------------------ RoPE

@pytest.mark.parametrize("pos", [1, 7, 513, 200000])
@pytest.mark.parametrize("j", [0, 1, 17, 63])
def test_rope_one_hot_is_a_rotation_of_its_pair(pos, j):
    # Head = 3 e_j (or 3 e_{j+64}); unit gain, eps 0: the norm gives
    # a = BF16(sqrt(128)) at that element; RoPE multiplies the pair
    # (x_j, x_{j+64}) read as x_j + i x_{j+64} by exp(i pos theta^(-2j/D)).
    theta = 10000.0
    ang = pos * theta ** (-2.0 * j / D)
    rot = np.exp(1j * ang)
    a = float(val(bits(math.sqrt(D))).ravel()[0])
    g = bits(np.ones(D))
    for partner in (0, 1):
        head = np.zeros(D)
        head[j + 64 * partner] = 3.0
        qkv = qkv_of(np.tile(head, (NQ, 1)), np.tile(head, (NKV, 1)), np.zeros((NKV, D)))
        q, k, _ = oracle.attn_prep(cfg(rope=1, eps=0.0, rope_theta=theta), qkv, [pos], g, g)
        z = a * rot * (1j if partner else 1.0)
        want = np.zeros(D)
        want[j], want[j + 64] = z.real, z.imag
        # compared as values: 0 cos - 0 sin may carry either sign of zero
        assert np.array_equal(val(q[0]), np.tile(bf.bf16(want), (NQ, 1))), (pos, j, partner)
        assert np.array_equal(val(k[0]), np.tile(bf.bf16(want), (NKV, 1)))


def test_rope_off_ignores_position_and_pos0_is_identity():
    qkv = rand_bits(9, (NQ + 2 * NKV) * D)[None]
    g1, g2 = rand_bits(10, D, 0.2), rand_bits(11, D, 0.2)
    base = oracle.attn_prep(cfg(rope=0), qkv, [0], g1, g2)
    for a, p in ((cfg(rope=0), 12345), (cfg(rope=1), 0)):
        got = oracle.attn_prep(a, qkv, [p], g1, g2)
        for x, y in zip(base, got):
            assert np.array_equal(x, y)


def test_rope_scores_depend_on_relative_position_only():
    # <R(p1) q, R(p2) k> = <R(p1 + s) q, R(p2 + s) k> up to the BF16
    # rounding of the rotated vectors.
    qkv = rand_bits(12, (NQ + 2 * NKV) * D)[None]
    g = bits(np.ones(D))
    a = cfg(rope=1)
    for p1, p2, s in ((40, 3, 1000), (700, 700, 65536), (5, 9, 123457)):
        qa, _, _ = oracle.attn_prep(a, qkv, [p1], g, g)
        _, ka, _ = oracle.attn_prep(a, qkv, [p2], g, g)
        qb, _, _ = oracle.attn_prep(a, qkv, [p1 + s], g, g)
        _, kb, _ = oracle.attn_prep(a, qkv, [p2 + s], g, g)
        for h in (0, 9, 31):
            da = val(qa[0, h]) @ val(ka[0, h // G])
            db = val(qb[0, h]) @ val(kb[0, h // G])
            assert abs(da - db) < 0.05 * D ** 0.5, (p1, p2, s, h, da, db)


def test_rope_preserves_pair_lengths():
    qkv = rand_bits(13, (NQ + 2 * NKV) * D)[None]
    g = bits(np.ones(D))
    q0, _, _ = oracle.attn_prep(cfg(rope=0), qkv, [0], g, g)
    q1, _, _ = oracle.attn_prep(cfg(rope=1), qkv, [98765], g, g)
    r0 = np.hypot(val(q0[0, :, :64]), val(q0[0, :, 64:]))
    r1 = np.hypot(val(q1[0, :, :64]), val(q1[0, :, 64:]))
    assert np.all(np.abs(r0 - r1) <= 2 ** -7 * r0 + 1e-30)


# ------------------------------------------------------------ decode attention

def sdpa_ref(q, keys, vals, sinks=None):
    """torch float64 SDPA over the linear list of attended positions.
    q [NQ, D]; keys, vals [n, NKV, D] (values); sinks [NQ] or None."""
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(keys.transpose(1, 0, 2))).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(np.ascontiguousarray(vals.transpose(1, 0, 2))).repeat_interleave(G, 0)[None]
    mask = None
    if sinks is not None:
        kt = torch.cat([kt, torch.zeros(1, NQ, 1, D, dtype=torch.float64)], 2)
        vt = torch.cat([vt, torch.zeros(1, NQ, 1, D, dtype=torch.float64)], 2)
        mask = torch.zeros(1, NQ, 1, kt.shape[2], dtype=torch.float64)
        mask[0, :, 0, -1] = torch.from_numpy(np.asarray(sinks, np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0, :, 0, :].numpy()


def ring(keys, vals, pos, slots):
    """Store positions 0..pos at slot p % slots (later positions overwrite)."""
    kc = np.zeros((slots, NKV, D), np.uint16)
    vc = np.zeros((slots, NKV, D), np.uint16)
    for p in range(pos + 1):
        kc[p % slots] = keys[p]
        vc[p % slots] = vals[p]
    return kc, vc


def decode(a, q, kc, vc, pos, sinks=None):
    return oracle.attn_decode(a, q[None], kc[None], vc[None], [pos], sinks)[0]


@pytest.mark.parametrize("with_sinks", [False, True])
def test_decode_matches_torch_sdpa(with_sinks):
    pos = 40
    q = rand_bits(20, NQ * D).reshape(NQ, D)
    keys = rand_bits(21, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    vals = rand_bits(22, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    sinks = synth.normal_f64(23, 7, 0, 2.0, NQ).astype(np.float32) if with_sinks else None
    got = decode(cfg(), q, keys, vals, pos, sinks)
    want = sdpa_ref(val(q), val(keys), val(vals), None if sinks is None else sinks.astype(np.float64))
    assert np.array_equal(got, bits(want))


@pytest.mark.parametrize("window,pos,slots", [(17, 100, 32), (513, 1500, 544), (513, 300, 544), (1, 9, 4)])
def test_decode_sliding_window_in_a_ring_matches_masked_sdpa(window, pos, slots):
    q = rand_bits(30, NQ * D).reshape(NQ, D)
    keys = rand_bits(31, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    vals = rand_bits(32, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    sinks = synth.normal_f64(33, 7, 0, 1.0, NQ).astype(np.float32)
    kc, vc = ring(keys, vals, pos, slots)
    got = decode(cfg(window=window), q, kc, vc, pos, sinks)
    lo = max(0, pos - window + 1)
    want = sdpa_ref(val(q), val(keys[lo:]), val(vals[lo:]), sinks.astype(np.float64))
    assert np.array_equal(got, bits(want))
    # the same positions stored linearly give the same bits
    assert np.array_equal(got, decode(cfg(window=window), q, keys, vals, pos, sinks))


def uniform_case(pos):
    """q = 0 (every score 0); V at position p = p - 150 in every element."""
    q = np.zeros((NQ, D), np.uint16)
    keys = rand_bits(40, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    vals = np.repeat(bits(np.arange(pos + 1) - 150.0)[:, None], NKV * D, 1).reshape(pos + 1, NKV, D)
    return q, keys, vals


@pytest.mark.parametrize("window,mean", [(9, 46.0), (10, 45.5), (8, 46.5), (0, -50.0)])
def test_decode_uniform_scores_average_the_window(window, mean):
    # pos 200: the window holds positions 201 - W .. 200, values 51 - W .. 50.
    q, keys, vals = uniform_case(200)
    got = decode(cfg(window=window), q, keys, vals, 200)
    assert np.all(got == bits(mean))


def test_decode_sink_in_the_denominator_only():
    # 9 equal scores of 0 and a sink of ln 9: weights 1 / 18 each, so the
    # output is half the window mean (46 / 2).
    q, keys, vals = uniform_case(200)
    sinks = np.full(NQ, math.log(9.0), np.float32)
    got = decode(cfg(window=9), q, keys, vals, 200, sinks)
    want = 46.0 * 9 / (9 + math.exp(float(sinks[0])))
    assert np.all(got == bits(want))
    very_low = np.full(NQ, -1e30, np.float32)
    assert np.array_equal(decode(cfg(window=9), q, keys, vals, 200, very_low),
                          decode(cfg(window=9), q, keys, vals, 200))


def test_decode_score_scale_is_inverse_sqrt_head_dim():
    # Two positions; q_h = 4 e_0; k_0 = 8 e_0, k_1 = 0; v_0 = 1, v_1 = 0:
    # out = sigmoid(32 / sqrt(128)).
    q = np.zeros((NQ, D))
    q[:, 0] = 4.0
    keys = np.zeros((2, NKV, D))
    keys[0, :, 0] = 8.0
    vals = np.zeros((2, NKV, D))
    vals[0] = 1.0
    got = decode(cfg(), bits(q), bits(keys), bits(vals), 1)
    assert np.all(got == bits(1.0 / (1.0 + math.exp(-32.0 / math.sqrt(D)))))


def test_decode_gqa_head_mapping():
    # V of KV head g is g + 1 everywhere, scores uniform: head h reads g = h // 8.
    pos = 30
    q = np.zeros((NQ, D), np.uint16)
    keys = rand_bits(41, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    vals = np.broadcast_to(bits(np.arange(NKV) + 1.0)[None, :, None], (pos + 1, NKV, D)).copy()
    got = decode(cfg(), q, keys, vals, pos)
    for h in range(NQ):
        assert np.all(got[h] == bits(h // G + 1.0)), h


def test_decode_one_dominant_key_returns_its_value():
    # s_7 - s_other = 2 * 256 / sqrt(128) ~ 45: the others weigh < 1e-19.
    pos = 20
    q = np.zeros((NQ, D))
    q[:, 0] = 16.0
    keys = np.zeros((pos + 1, NKV, D))
    keys[:, :, 0] = -16.0
    keys[7, :, 0] = 16.0
    vals = rand_bits(42, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    got = decode(cfg(), bits(q), bits(keys), vals, pos)
    assert np.array_equal(got, np.repeat(vals[7], G, 0))


def test_decode_batch_rows_are_independent():
    pos = [3, 50, 0]
    qs = rand_bits(43, 3 * NQ * D).reshape(3, NQ, D)
    kc = rand_bits(44, 3 * 64 * NKV * D).reshape(3, 64, NKV, D)
    vc = rand_bits(45, 3 * 64 * NKV * D).reshape(3, 64, NKV, D)
    out = oracle.attn_decode(cfg(window=5), qs, kc, vc, pos)
    for t in range(3):
        assert np.array_equal(out[t], decode(cfg(window=5), qs[t], kc[t], vc[t], pos[t]))


def test_decode_scores_beyond_exp_range_stay_finite():
    # s = 90 * 90 / sqrt(128) ~ 716 > ln(DBL_MAX): the softmax must shift by
    # its maximum, as softmax(s) = softmax(s - c) for any c.
    pos = 4
    q = np.zeros((NQ, D))
    q[:, 0] = 90.0
    keys = np.zeros((pos + 1, NKV, D))
    keys[2, :, 0] = 90.0
    vals = rand_bits(46, (pos + 1) * NKV * D).reshape(pos + 1, NKV, D)
    sinks = np.full(NQ, 700.0, np.float32)
    got = decode(cfg(), bits(q), bits(keys), vals, pos, sinks)
    assert np.array_equal(got, np.repeat(vals[2], G, 0))

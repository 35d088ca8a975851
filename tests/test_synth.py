"""The seeded input generator: known answers, moments, encoders, layout."""
import os

import numpy as np

import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for r in rows:
        v = [int(t, 16) for t in r]
        assert list(synth.philox4x32_10(v[:4], v[4:6])) == v[6:10]


def test_normal_moments_and_determinism():
    z = synth.normal_f64(123, 0, 0, 1.0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    assert np.array_equal(z, synth.normal_f64(123, 0, 0, 1.0, 1 << 20))
    assert not np.array_equal(z[:100], synth.normal_f64(124, 0, 0, 1.0, 100))
    # counter-based: a prefix is the prefix of a longer draw
    assert np.array_equal(synth.normal_f64(123, 0, 0, 1.0, 101), z[:101])


def test_e2m1_encoder_is_nearest_even():
    rng = np.random.default_rng(0)
    ts = np.concatenate([rng.uniform(-7, 7, 4000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.0]])
    for t in ts:
        c = synth.lib().synth_e2m1_encode(float(t))
        d = np.abs(bf.E2M1[:8] - min(abs(t), 6.0))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c & 7 == want, t
        assert (c >> 3) == (1 if (t < 0 and want != 0) else 0)


def test_e4m3_encoder_is_nearest_even():
    vals = bf.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    rng = np.random.default_rng(1)
    ts = np.concatenate([rng.uniform(0, 460, 2000), np.exp(rng.uniform(-14, 6, 2000)),
                         (vals[1:] + vals[:-1]) / 2])
    for t in ts:
        c = synth.lib().synth_e4m3_encode_pos(float(t))
        d = np.abs(vals - min(t, 448.0))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, t


def test_layer_shapes_and_zipf_spread():
    L = synth.make_layer(0, hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6, bias="zipf")
    assert L["w_gate"].shape == (32, 64, 256 // 16 * 9)
    assert L["w_down"].shape == (32, 256, 64 // 16 * 9)
    assert L["w_scale"].shape == (32, 3) and L["router_w"].shape == (32, 256)
    b = synth.zipf_offset(256)
    assert abs(float(b.mean())) < 1e-5
    ln_rank = np.sort(-(b.astype(np.float64) - b.max()) / (0.6 * 1.1))
    assert np.allclose(ln_rank, np.log(np.arange(1, 257)), atol=1e-5)

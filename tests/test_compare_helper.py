"""CPU checks of the GPU tests' acceptance helper (tests/gpu_util.py): on a
token the oracle flags as a near tie, a selection the tie allows passes
and others fail.  The "GPU" results here are made by the oracle itself."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_flagged, compare


def _layer(biases, k):
    L = synth.make_layer(0, hidden=64, inter=32, shared_inter=32, n_experts=len(biases), top_k=k)
    L["router_b"] = np.asarray(biases, np.float32)
    return L


# experts 1, 4 at 5; expert 3 at 0 (k-th) and expert 5 at -3.6e-5 tie
# within 1e-5 in score; the others at -5
TIE = [-5, 5, -5, 0, 5, -3.6e-5, -5, -5]


def _run(L, x, idx):
    r = oracle.moe_tokens(L, x, forced_idx=np.asarray([idx], np.int32))
    return r["out"], r["idx"], r["w"].astype(np.float32)


def test_flagged_token_accepts_either_tied_set():
    L = _layer(TIE, 3)
    x = np.zeros((1, 64), np.uint16)
    for idx in ([4, 1, 3], [4, 1, 5]):
        out, gi, gw = _run(L, x, idx)
        _, st = compare(L, x, out, gi, gw)
        assert st["flagged"] == 1


@pytest.mark.parametrize("idx", [[4, 1, 0], [4, 3, 5], [4, 1, 1]])
def test_flagged_token_rejects_sets_the_tie_does_not_allow(idx):
    # a loser (expert 0), a dropped clear winner (expert 1), a repeat
    L = _layer(TIE, 3)
    x = np.zeros((1, 64), np.uint16)
    ref = oracle.moe_tokens(L, x)
    forced = oracle.moe_tokens(L, x, forced_idx=np.asarray([idx], np.int32))
    with pytest.raises(AssertionError):
        check_flagged(ref["logits"][0], forced["idx"][0], forced["w"][0], idx, forced["w"][0], 3)


def test_flagged_token_rejects_wrong_weights():
    L = _layer(TIE, 3)
    x = np.zeros((1, 64), np.uint16)
    ref = oracle.moe_tokens(L, x)
    idx = [4, 1, 5]
    forced = oracle.moe_tokens(L, x, forced_idx=np.asarray([idx], np.int32))
    w = forced["w"][0].copy()
    w[2] *= 1.001
    with pytest.raises(AssertionError):
        check_flagged(ref["logits"][0], forced["idx"][0], forced["w"][0], idx, w, 3)


def test_unflagged_token_needs_the_exact_set():
    L = _layer([-5, 5, -5, 0, 5, -1, -5, -5], 3)
    x = np.zeros((1, 64), np.uint16)
    out, gi, gw = _run(L, x, [4, 1, 5])
    with pytest.raises(AssertionError):
        compare(L, x, out, gi, gw)


def _fake_layer_out(L, x):
    r = oracle.moe_tokens(L, x)
    return r, r["out"].copy()


def test_one_ulp_allowance_only_where_an_ulp_exceeds_the_bar():
    # A dense layer: oracle outputs; move one element of magnitude >= 2 by
    # one BF16 ulp (allowed, it is a rounding-midpoint flip), by two ulps
    # (refused), and one element below 2 by one ulp of 0.0078 (within 1e-2).
    L = synth.make_layer(0, hidden=256, inter=0, shared_inter=2112, n_experts=0, sigma=0.1)
    x = synth.tokens(64, 256, stream=3)
    ref, out = _fake_layer_out(L, x)
    v = oracle.bf16_to_f64(ref["out"])
    big = np.argwhere(np.abs(v) >= 2.0)
    if len(big) == 0:
        pytest.skip("no output of magnitude >= 2 in this sample")
    t, j = big[0]
    one = out.copy()
    one[t, j] += 1  # next BF16 magnitude: one ulp
    compare(L, x, one, None, None, ref=ref)
    two = out.copy()
    two[t, j] += 2
    with pytest.raises(AssertionError):
        compare(L, x, two, None, None, ref=ref)


def test_one_ulp_allowance_is_rare():
    # Flipping many large elements by one ulp is a systematic error.
    L = synth.make_layer(0, hidden=256, inter=0, shared_inter=2112, n_experts=0, sigma=0.1)
    x = synth.tokens(64, 256, stream=3)
    ref, out = _fake_layer_out(L, x)
    v = oracle.bf16_to_f64(ref["out"])
    big = np.abs(v) >= 2.0
    if np.count_nonzero(big) < 3:
        pytest.skip("too few outputs of magnitude >= 2 in this sample")
    many = out.copy()
    many[big] += 1
    with pytest.raises(AssertionError):
        compare(L, x, many, None, None, ref=ref)

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

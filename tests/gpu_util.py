"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle to the acceptance bar of the layer:
  - selected expert sets bit-exact per token, except tokens the oracle flags
    (6th/7th sigmoid score gap < 1e-5).  For those, every expert whose score
    clears the (k+1)-th by more than 1e-5 must be selected, every selected
    expert must score within 1e-5 of the k-th, and the outputs and weights
    are compared with the oracle re-run on the GPU's selection;
  - combine weights within 1e-5 relative of the oracle's (FP32 sigmoid and
    sum against FP64);
  - outputs: rel-L2 <= 2e-3 over the whole [B][H] block and max-abs <= 1e-2,
    except that an element may differ from the oracle's by one BF16 ulp
    where one ulp exceeds 1e-2 (oracle values of magnitude >= 2, e.g. the
    wide dense layers' outputs): a sum accumulated in FP32 and rounded
    once can land on the other side of a BF16 rounding midpoint than the
    FP64 sum, and 1e-2 is finer than the format there.  Such flips are
    rare (the FP32 sum must lie within its own rounding error of a
    midpoint), so at most 1 in 10^4 elements may use this allowance.
"""
import sys

import numpy as np
import torch

import oracle

REL_L2 = 2e-3
MAX_ABS = 1e-2
ULP_FLIP_FRACTION = 1e-4


def bf16_ulp(v):
    """One BF16 ulp at each value (normal range: 2^(exponent - 7))."""
    m, e = np.frexp(np.abs(np.asarray(v, np.float64)))
    return np.ldexp(1.0, e - 8)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).cuda()


def from_dev_bits(t):
    return t.cpu().numpy().view(np.uint16)


def wait_status(ws):
    """The wait status word of the last decode call on workspace ws (0:
    every bounded wait inside its kernels saw what it waited for)."""
    import w4a16_routed_expert_sigmoid_amd as moe
    s = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    moe.moe_decode_wait_status(ws, s)
    return int(s.item())


def bf16_f64(bits):
    return oracle.bf16_to_f64(bits)


def check_flagged(logits, forced_idx, forced_w, gidx, gw, k, what=""):
    """A flagged token (near tie at the k-th score): the GPU's set gidx must
    be one the tie allows, and its weights gw those the oracle gives that set
    (forced_idx / forced_w: the oracle re-run with gidx forced)."""
    E = len(logits)
    s = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
    order = sorted(range(E), key=lambda e: (-logits[e], e))
    sk = s[order[k - 1]]
    sk1 = s[order[k]] if E > k else -np.inf
    sel = [int(e) for e in gidx]
    assert len(set(sel)) == k and all(0 <= e < E for e in sel), f"{what}: {sel}"
    must = {e for e in range(E) if s[e] > sk1 + 1e-5}
    assert must <= set(sel), f"{what}: missing clear winners {sorted(must - set(sel))}"
    assert all(s[e] >= sk - 1e-5 for e in sel), f"{what}: a selected expert scores below the tie"
    wmap = dict(zip([int(e) for e in forced_idx], [float(v) for v in forced_w]))
    for e, w in zip(sel, [float(v) for v in gw]):
        assert abs(w - wmap[e]) <= 1e-5 * abs(wmap[e]) + 1e-7, f"{what}: expert {e} weight"


def compare(layer, x, gpu_out, gpu_idx, gpu_w, ref=None, what=""):
    """Assert the acceptance bar; returns (ref, stats).  The oracle runs on
    every host thread (bit-identical to one thread)."""
    if ref is None:
        ref = oracle.moe_tokens(layer, x, threads=None)
    assert ref["nan_tokens"] == 0
    out_ref = ref["out"]
    E = layer["n_experts"]
    flagged = 0
    if E > 0:
        k = layer["top_k"]
        flag_t = [t for t in range(x.shape[0]) if ref["flag"][t]]
        flagged = len(flag_t)
        for t in range(x.shape[0]):
            if ref["flag"][t]:
                continue
            gs, rs = set(gpu_idx[t].tolist()), set(ref["idx"][t].tolist())
            assert gs == rs, f"{what} token {t}: gpu {sorted(gs)} oracle {sorted(rs)}"
            wmap = dict(zip(ref["idx"][t].tolist(), ref["w"][t].tolist()))
            for e, w in zip(gpu_idx[t].tolist(), gpu_w[t].tolist()):
                assert abs(w - wmap[e]) <= 1e-5 * abs(wmap[e]) + 1e-7, f"{what} token {t} expert {e}"
        if flag_t:
            log(f"  {what}: {flagged} of {x.shape[0]} tokens flagged (near tie at the k-th score)")
            sub = np.array(flag_t)
            forced = oracle.moe_tokens(layer, x[sub], forced_idx=gpu_idx[sub], threads=None)
            out_ref = out_ref.copy()
            for i, t in enumerate(flag_t):
                check_flagged(ref["logits"][t], forced["idx"][i], forced["w"][i], gpu_idx[t], gpu_w[t], k,
                              f"{what} token {t} (flagged)")
                out_ref[t] = forced["out"][i]
    st = check_outputs(gpu_out, out_ref, what)
    st["flagged"] = flagged
    return ref, st


def check_outputs(gpu_out, out_ref, what=""):
    """The output bar on BF16 bits (see the module docstring); returns stats."""
    o = bf16_f64(gpu_out)
    r = bf16_f64(out_ref)
    assert np.all(np.isfinite(o)), what
    rel = float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-30))
    d = np.abs(o - r)
    mx = float(np.max(d))
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    over = d > MAX_ABS
    n_over = int(np.count_nonzero(over))
    if n_over:
        assert np.all(d[over] <= bf16_ulp(r[over])), \
            f"{what}: max-abs {mx:.3e}, more than one BF16 ulp at {np.argwhere(over & (d > bf16_ulp(r)))[:4]}"
        assert n_over <= ULP_FLIP_FRACTION * d.size, f"{what}: {n_over} elements one ulp (> 1e-2) apart"
        log(f"  {what}: {n_over} of {d.size} elements one BF16 ulp (> 1e-2) from the oracle")
    return dict(rel_l2=rel, max_abs=mx, ulp_flips_over_1e2=n_over, bit_exact=float(np.mean(gpu_out == out_ref)))

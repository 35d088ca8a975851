"""Brute-force dense MoE, written independently of the oracle, for its pins.

It evaluates *every* expert densely and mixes them with a gate vector that
is zero outside the selected set, instead of visiting only the selected
experts.  Nothing here is shared with the oracle: weights are decoded with
torch's float8_e4m3fn conversion and the E2M1 table from the OCP MX
specification (tests/golden/e2m1_ocp.txt), and BF16 rounding is done as
round-to-odd FP64->FP32 followed by torch's FP32->BF16 round-to-nearest-even
(a correct single rounding because FP32 keeps 16 spare bits).
"""
import os

import numpy as np
import torch

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table():
    vals = {}
    with open(os.path.join(_GOLDEN, "e2m1_ocp.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)], dtype=np.float64)


E2M1 = e2m1_table()


def e4m3_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def bf16_bits_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def bf16(v):
    """FP64 -> nearest-even BF16 value (as FP64), via round-to-odd FP32."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    back = f.astype(np.float64)
    inexact = (back != v) & np.isfinite(v)
    over = inexact & (np.abs(back) > np.abs(v))
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    bits = f.view(np.uint32).copy()
    bits[inexact] |= np.uint32(1)
    f = bits.view(np.float32)
    return torch.from_numpy(np.ascontiguousarray(f)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_bits(v):
    t = torch.from_numpy(np.ascontiguousarray(bf16(v), dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def decode_matrix(m, rows, cols, wtype, scale=1.0):
    """Weights -> FP64 [rows, cols].  NVFP4 in the GGUF-like 9-byte blocks."""
    if wtype == "bf16":
        return bf16_bits_to_f64(m).reshape(rows, cols)
    blk = np.asarray(m, dtype=np.uint8).reshape(rows, cols // 16, 9)
    s = e4m3_decode(blk[:, :, 0])
    nib = blk[:, :, 1:]
    codes = np.concatenate([nib & 15, nib >> 4], axis=2)  # element j, then j+8
    return (E2M1[codes] * s[:, :, None] * scale).reshape(rows, cols)


def _ffn(Wg, Wu, Wd, xn):
    g = bf16(Wg @ xn)
    u = bf16(Wu @ xn)
    h = bf16(g / (1.0 + np.exp(-g)) * u)
    return bf16(Wd @ h)


def dense_moe(layer, x_bits, forced=None):
    """All tokens x [T, H] -> (out bits [T, H], selected sets [T] of frozensets)."""
    H, I, Is, E = layer["hidden"], layer["inter"], layer["shared_inter"], layer["n_experts"]
    k, wt = layer["top_k"], layer["wtype"]
    ws = layer.get("w_scale")
    Wr = bf16_bits_to_f64(layer["router_w"]).reshape(E, H) if E else None
    b = np.zeros(E) if layer.get("router_b") is None else np.asarray(layer["router_b"], np.float64)
    experts = []
    for e in range(E):
        sg, su, sd = (ws[e] if ws is not None else (1.0, 1.0, 1.0))
        experts.append((decode_matrix(layer["w_gate"][e], I, H, wt, sg),
                        decode_matrix(layer["w_up"][e], I, H, wt, su),
                        decode_matrix(layer["w_down"][e], H, I, wt, sd)))
    shared = None
    if Is:
        ss = layer.get("sh_scale")
        sg, su, sd = (ss if ss is not None else (1.0, 1.0, 1.0))
        shared = (decode_matrix(layer["sh_gate"], Is, H, wt, sg),
                  decode_matrix(layer["sh_up"], Is, H, wt, su),
                  decode_matrix(layer["sh_down"], H, Is, wt, sd))
    xs = bf16_bits_to_f64(x_bits).reshape(-1, H)
    outs, sets = [], []
    for t, x in enumerate(xs):
        if layer.get("norm_gain") is not None:
            g = bf16_bits_to_f64(layer["norm_gain"])
            xn = bf16(x / np.sqrt(np.mean(x * x) + layer["eps"]) * g)
        else:
            xn = x
        acc = np.zeros(H)
        if E:
            logits = Wr @ xn + b
            s = 1.0 / (1.0 + np.exp(-logits))
            order = np.lexsort((np.arange(E), -logits))  # logit desc, index asc
            sel = order[:k] if forced is None else np.asarray(forced[t])
            gate = np.zeros(E)
            gate[sel] = s[sel] / s[sel].sum()
            Y = np.stack([_ffn(*experts[e], xn) for e in range(E)])  # every expert, densely
            acc = gate @ Y
            sets.append(frozenset(int(v) for v in sel))
        if shared is not None:
            acc = acc + _ffn(*shared, xn)
        o = bf16(acc)
        if layer.get("residual"):
            o = bf16(x + o)
        outs.append(bf16_bits(o))
    return np.stack(outs), sets

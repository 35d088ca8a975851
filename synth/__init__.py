"""Seeded synthetic inputs for the W4A16 sigmoid-routed MoE layer.

Serves both the CPU oracle and the GPU path.  Holds none of the layer's
arithmetic: it draws N(0, sigma) values with the counter-based Philox4x32-10
generator, rounds them to BF16 or quantises them to NVFP4, and writes the
bytes in the orders below.  ``synth.c`` documents the generator and the
quantiser.

Workload recipe (the pages' shapes: hidden 2048, 256 routed experts, top-6,
one shared expert; intermediate 512 is an assumption the pages leave open):
  weights   seed = 1000 + layer; router BF16(N(0, 0.02)); expert and shared
            matrices N(0, 0.02), BF16 or NVFP4-quantised (GGUF-like order)
  tokens    seed 42, BF16(N(0, 1))
  offset    Zipf(1.1) rank offset, permutation seed 7, beta 0.6
  gains     BF16(1 + 0.02 N(0, 1)) per layer (pre-norm layers only)
Stream ids (Philox counter words 2 and 3): word 2 = 0, word 3 = tensor id:
  gate/up/down of expert e = 4e + 0/1/2; shared gate/up/down = 0x100000 + 0/1/2;
  router = 0x200000; gain = 0x300000; tokens use word 2 = stream, word 3 = 0x400000.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
# MOE_HOST_LIB_DIR: load the library from another directory (the CPU tests
# point it at builds with the address and undefined-behaviour sanitizers).
_LIB = os.path.join(os.environ.get("MOE_HOST_LIB_DIR") or _HERE, "libsynth.so")
_lib = None

WEIGHT_SEED_BASE = 1000
TOKEN_SEED = 42
ZIPF_SEED = 7
TID_SHARED = 0x100000
TID_ROUTER = 0x200000
TID_GAIN = 0x300000
TID_TOKENS = 0x400000


def build():
    """Compile synth.c with gcc into synth/libsynth.so (always rebuilds)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, u32, i64, dbl, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_normal_f64.argtypes = [u64, u32, u32, dbl, i64, vp]
        L.synth_normal_bf16.argtypes = [u64, u32, u32, dbl, i64, vp]
        L.synth_gain_bf16.argtypes = [u64, u32, u32, dbl, i64, vp]
        L.synth_quantize_nvfp4.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
        L.synth_nvfp4_normal.argtypes = [u64, u32, u32, dbl, i64, i64, ctypes.c_int, vp, vp]
        L.synth_nvfp4_normal_stack.argtypes = [u64, u32, u32, u32, i64, dbl, i64, i64, ctypes.c_int, vp, vp, i64]
        L.synth_nvfp4_normal_stack.restype = ctypes.c_int
        L.synth_bf16_normal_stack.argtypes = [u64, u32, u32, u32, i64, dbl, i64, vp]
        L.synth_zipf_offset.argtypes = [u64, ctypes.c_int32, dbl, dbl, vp]
        L.synth_e2m1_encode.argtypes = [dbl]
        L.synth_e2m1_encode.restype = ctypes.c_int
        L.synth_e4m3_encode_pos.argtypes = [dbl]
        L.synth_e4m3_encode_pos.restype = ctypes.c_int
        _lib = L
    return _lib


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    o = np.empty(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return o


def normal_f64(seed, a, b, sigma, n):
    out = np.empty(n, dtype=np.float64)
    lib().synth_normal_f64(seed, a, b, sigma, n, out.ctypes.data)
    return out


def normal_bf16(seed, a, b, sigma, n):
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(seed, a, b, sigma, n, out.ctypes.data)
    return out


def quantize_nvfp4(w, pow2_tensor_scale=False):
    """Real matrix [rows, cols] -> (GGUF-like bytes [rows, cols/16*9], FP32 tensor scale)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    rows, cols = w.shape
    assert cols % 16 == 0
    out = np.empty((rows, cols // 16 * 9), dtype=np.uint8)
    s = np.empty(1, dtype=np.float32)
    lib().synth_quantize_nvfp4(w.ctypes.data, rows, cols, int(pow2_tensor_scale), out.ctypes.data, s.ctypes.data)
    return out, float(s[0])


def nvfp4_stack(seed, tid0, tid_stride, n_mats, rows, cols, sigma=0.02, pow2_tensor_scale=False):
    """n_mats NVFP4 matrices -> (uint8 [n_mats, rows, cols/16*9], float32 [n_mats])."""
    out = np.empty((n_mats, rows, cols // 16 * 9), dtype=np.uint8)
    sc = np.empty(n_mats, dtype=np.float32)
    rc = lib().synth_nvfp4_normal_stack(seed, 0, tid0, tid_stride, n_mats, sigma, rows, cols,
                                         int(pow2_tensor_scale), out.ctypes.data, sc.ctypes.data, 1)
    if rc:
        raise MemoryError("synth: out of memory")
    return out, sc


def bf16_stack(seed, tid0, tid_stride, n_mats, rows, cols, sigma=0.02):
    out = np.empty((n_mats, rows, cols), dtype=np.uint16)
    lib().synth_bf16_normal_stack(seed, 0, tid0, tid_stride, n_mats, sigma, rows * cols, out.ctypes.data)
    return out


def zipf_offset(n_experts, alpha=1.1, beta=0.6, seed=ZIPF_SEED):
    out = np.empty(n_experts, dtype=np.float32)
    lib().synth_zipf_offset(seed, n_experts, alpha, beta, out.ctypes.data)
    return out


def tokens(batch, hidden, stream=0, seed=TOKEN_SEED, sigma=1.0):
    """BF16(N(0, sigma)) token vectors [batch, hidden] as bf16 bits."""
    return normal_bf16(seed, stream, TID_TOKENS, sigma, batch * hidden).reshape(batch, hidden)


def gain(hidden, layer_id, sigma=0.02):
    out = np.empty(hidden, dtype=np.uint16)
    lib().synth_gain_bf16(WEIGHT_SEED_BASE + layer_id, 0, TID_GAIN, sigma, hidden, out.ctypes.data)
    return out


def make_layer(layer_id=0, hidden=2048, inter=512, shared_inter=512, n_experts=256, top_k=6,
               wtype="nvfp4", sigma=0.02, bias="zero", norm=False, residual=False,
               eps=float(np.float32(1e-6)), pow2_tensor_scale=False):
    """One layer's weights as the dict the oracle and the GPU binding read.

    bias: 'zero' | 'zipf' | 'none' | float32 array [E].  n_experts = 0 gives a
    dense SwiGLU layer (the shared expert alone, of width shared_inter).
    """
    seed = WEIGHT_SEED_BASE + layer_id
    H, I, Is, E = hidden, inter, shared_inter, n_experts
    L = dict(hidden=H, inter=I, shared_inter=Is, n_experts=E, top_k=top_k if E > 0 else 0,
             wtype=wtype, eps=eps, residual=int(residual), norm_gain=None,
             router_w=None, router_b=None, w_gate=None, w_up=None, w_down=None, w_scale=None,
             sh_gate=None, sh_up=None, sh_down=None, sh_scale=None)
    if norm:
        L["norm_gain"] = gain(H, layer_id)
    if E > 0:
        L["router_w"] = normal_bf16(seed, 0, TID_ROUTER, sigma, E * H).reshape(E, H)
        if isinstance(bias, str):
            if bias == "zero":
                L["router_b"] = np.zeros(E, dtype=np.float32)
            elif bias == "zipf":
                L["router_b"] = zipf_offset(E)
            elif bias == "none":
                L["router_b"] = None
            else:
                raise ValueError(bias)
        else:
            L["router_b"] = np.ascontiguousarray(bias, dtype=np.float32)
        if wtype == "nvfp4":
            L["w_scale"] = np.empty((E, 3), dtype=np.float32)
            for p, key, (r, c) in ((0, "w_gate", (I, H)), (1, "w_up", (I, H)), (2, "w_down", (H, I))):
                m, s = nvfp4_stack(seed, p, 4, E, r, c, sigma, pow2_tensor_scale)
                L[key] = m
                L["w_scale"][:, p] = s
        else:
            L["w_gate"] = bf16_stack(seed, 0, 4, E, I, H, sigma)
            L["w_up"] = bf16_stack(seed, 1, 4, E, I, H, sigma)
            L["w_down"] = bf16_stack(seed, 2, 4, E, H, I, sigma)
    if Is > 0:
        if wtype == "nvfp4":
            L["sh_scale"] = np.empty(3, dtype=np.float32)
            for p, key, (r, c) in ((0, "sh_gate", (Is, H)), (1, "sh_up", (Is, H)), (2, "sh_down", (H, Is))):
                m, s = nvfp4_stack(seed, TID_SHARED + p, 0, 1, r, c, sigma, pow2_tensor_scale)
                L[key] = m[0]
                L["sh_scale"][p] = s[0]
        else:
            L["sh_gate"] = bf16_stack(seed, TID_SHARED + 0, 0, 1, Is, H, sigma)[0]
            L["sh_up"] = bf16_stack(seed, TID_SHARED + 1, 0, 1, Is, H, sigma)[0]
            L["sh_down"] = bf16_stack(seed, TID_SHARED + 2, 0, 1, H, Is, sigma)[0]
    return L

"""CPU oracle of the W4A16 sigmoid-routed MoE layer and of the decode
attention beside it (FP64, plain C).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark, never by the product package.  This
wrapper only marshals numpy arrays into ``oracle.c``; the arithmetic and its
page citations live there.

A layer is a dict of numpy arrays with these keys (the convention the input
generator in ``synth`` writes):
  hidden, inter, shared_inter, n_experts, top_k, wtype ('bf16' | 'nvfp4'),
  eps (float), residual (0/1),
  norm_gain  uint16 [H] bf16 bits or None,
  router_w   uint16 [E, H], router_b float32 [E] or None,
  w_gate/w_up  NVFP4: uint8 [E, I, H/16*9] (GGUF-like blocks) | BF16: uint16 [E, I, H]
  w_down       NVFP4: uint8 [E, H, I/16*9]                    | BF16: uint16 [E, H, I]
  w_scale    float32 [E, 3] (NVFP4 tensor scales: gate, up, down) or None
  sh_gate/sh_up/sh_down (shared expert, same layouts without E), sh_scale float32 [3]
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# MOE_HOST_LIB_DIR: load the library from another directory (the CPU tests
# point it at builds with the address and undefined-behaviour sanitizers).
_LIB = os.path.join(os.environ.get("MOE_HOST_LIB_DIR") or _HERE, "liboracle.so")
_lib = None


def build():
    """Compile oracle.c with gcc into oracle/liboracle.so (always rebuilds)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-shared", "-fPIC", "-pthread",
                           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


class _Layer(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("wtype", ctypes.c_int32),
        ("norm_eps", ctypes.c_double), ("residual", ctypes.c_int32),
        ("norm_gain", ctypes.c_void_p), ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("w_scale", ctypes.c_void_p),
        ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
        ("sh_scale", ctypes.c_void_p),
    ]


class _Attn(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rope", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("norm_eps", ctypes.c_double)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int32]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_int32]
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [ctypes.c_double]
        L.oracle_bf16_round_array.restype = None
        L.oracle_bf16_round_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_decode_nvfp4.restype = ctypes.c_int64
        L.oracle_decode_nvfp4.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_double, ctypes.c_void_p]
        L.oracle_gemv_nvfp4.restype = ctypes.c_int64
        L.oracle_gemv_nvfp4.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        L.oracle_attn_prep.restype = None
        L.oracle_attn_prep.argtypes = [ctypes.POINTER(_Attn), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_attn_decode.restype = None
        L.oracle_attn_decode.argtypes = [ctypes.POINTER(_Attn), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_moe_tokens.restype = ctypes.c_int32
        L.oracle_moe_tokens.argtypes = [ctypes.POINTER(_Layer), ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_moe_tokens_mt.restype = ctypes.c_int32
        L.oracle_moe_tokens_mt.argtypes = L.oracle_moe_tokens.argtypes + [ctypes.c_int32]
        _lib = L
    return _lib


def host_threads():
    """Threads the oracle uses by default: the CPUs this process may run on,
    at most 16 (a one-GPU machine's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def e2m1_value(code):
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(code):
    return lib().oracle_e4m3_value(int(code))


def bf16_value(bits):
    return lib().oracle_bf16_value(int(bits))


def bf16_round(v):
    """FP64 -> BF16 bits, one round-to-nearest-even."""
    return lib().oracle_bf16_round(float(v))


def bf16_round_array(v):
    """Vector form of bf16_round: FP64 array -> BF16 bits (same shape)."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_to_f64(bits):
    """Vector form of bf16_value (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_nvfp4(src, rows, cols, tensor_scale):
    """GGUF-like NVFP4 bytes -> (FP64 [rows, cols], number of NaN scale bytes)."""
    src = np.ascontiguousarray(src, dtype=np.uint8)
    assert src.size == rows * (cols // 16) * 9
    out = np.empty((rows, cols), dtype=np.float64)
    nan = lib().oracle_decode_nvfp4(src.ctypes.data, rows, cols, float(tensor_scale), out.ctypes.data)
    return out, int(nan)


def gemv_nvfp4(src, rows, cols, tensor_scale, x):
    """Dense NVFP4 projection of T tokens: GGUF-like bytes [rows, cols],
    x [T, cols] BF16 bits -> (y [T, rows] BF16 bits, NaN scale bytes met)."""
    src = np.ascontiguousarray(src, dtype=np.uint8)
    assert src.size == rows * (cols // 16) * 9
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, cols)
    y = np.empty((x.shape[0], rows), dtype=np.uint16)
    nan = lib().oracle_gemv_nvfp4(src.ctypes.data, rows, cols, float(tensor_scale), x.ctypes.data, x.shape[0],
                                  y.ctypes.data)
    return y, int(nan)


def _attn(a):
    return _Attn(n_q=a["n_q"], n_kv=a["n_kv"], head_dim=a["head_dim"], window=a.get("window", 0),
                 rope=int(a.get("rope", 0)), rope_theta=float(a.get("rope_theta", 10000.0)),
                 norm_eps=float(a.get("eps", np.float32(1e-6))))


def attn_prep(a, qkv, pos, q_gain, k_gain):
    """Q/K norm + RoPE of T tokens: qkv [T, (n_q + 2 n_kv) * D] BF16 bits,
    pos [T] -> (q [T, n_q, D], k [T, n_kv, D], v [T, n_kv, D]) BF16 bits.
    a: dict(n_q, n_kv, head_dim, window, rope, rope_theta, eps)."""
    D, nq, nkv = a["head_dim"], a["n_q"], a["n_kv"]
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16).reshape(-1, (nq + 2 * nkv) * D)
    T = qkv.shape[0]
    qg = np.ascontiguousarray(q_gain, dtype=np.uint16)
    kg = np.ascontiguousarray(k_gain, dtype=np.uint16)
    q = np.empty((T, nq, D), np.uint16)
    k = np.empty((T, nkv, D), np.uint16)
    v = np.empty((T, nkv, D), np.uint16)
    s = _attn(a)
    for t in range(T):
        lib().oracle_attn_prep(ctypes.byref(s), qkv[t].ctypes.data, int(pos[t]), qg.ctypes.data, kg.ctypes.data,
                               q[t].ctypes.data, k[t].ctypes.data, v[t].ctypes.data)
    return q, k, v


def attn_decode(a, q, k_cache, v_cache, pos, sinks=None):
    """Decode attention of T tokens: q [T, n_q, D] BF16 bits; k_cache,
    v_cache [T, slots, n_kv, D] BF16 bits (one cache per token's sequence);
    pos [T]; sinks [n_q] FP32 or None -> out [T, n_q, D] BF16 bits."""
    D, nq = a["head_dim"], a["n_q"]
    q = np.ascontiguousarray(q, dtype=np.uint16).reshape(-1, nq * D)
    T = q.shape[0]
    kc = np.ascontiguousarray(k_cache, dtype=np.uint16)
    vc = np.ascontiguousarray(v_cache, dtype=np.uint16)
    slots = kc.shape[1]
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float32)
    out = np.empty((T, nq, D), np.uint16)
    s = _attn(a)
    for t in range(T):
        lib().oracle_attn_decode(ctypes.byref(s), q[t].ctypes.data, kc[t].ctypes.data, vc[t].ctypes.data, slots,
                                 int(pos[t]), None if sk is None else sk.ctypes.data, out[t].ctypes.data)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_layer(layer, keep):
    def arr(key, dtype):
        v = layer.get(key)
        if v is None:
            return None
        a = np.ascontiguousarray(v, dtype=dtype)
        keep.append(a)
        return a

    wdt = np.uint16 if layer["wtype"] == "bf16" else np.uint8
    s = _Layer()
    s.hidden, s.inter, s.shared_inter = layer["hidden"], layer["inter"], layer["shared_inter"]
    s.n_experts, s.top_k = layer["n_experts"], layer["top_k"]
    s.wtype = 0 if layer["wtype"] == "bf16" else 1
    s.norm_eps = float(layer.get("eps", 0.0))
    s.residual = int(layer.get("residual", 0))
    s.norm_gain = _ptr(arr("norm_gain", np.uint16))
    s.router_w = _ptr(arr("router_w", np.uint16))
    s.router_b = _ptr(arr("router_b", np.float32))
    s.w_gate = _ptr(arr("w_gate", wdt))
    s.w_up = _ptr(arr("w_up", wdt))
    s.w_down = _ptr(arr("w_down", wdt))
    s.w_scale = _ptr(arr("w_scale", np.float32))
    s.sh_gate = _ptr(arr("sh_gate", wdt))
    s.sh_up = _ptr(arr("sh_up", wdt))
    s.sh_down = _ptr(arr("sh_down", wdt))
    s.sh_scale = _ptr(arr("sh_scale", np.float32))
    return s


def moe_tokens(layer, x, forced_idx=None, threads=1):
    """Run T tokens x [T, H] (bf16 bits) through the layer.

    Returns dict(out [T,H] uint16, idx [T,k] int32, w [T,k] f64, flag [T] int32,
    logits [T,E] f64, nan_tokens int).  forced_idx [T,k] replaces the selection.
    threads > 1 spreads the tokens over host threads (one owner per token, so
    the results are bit-identical to threads == 1); None = host_threads().
    """
    keep = []
    s = _as_layer(layer, keep)
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, layer["hidden"])
    T = x.shape[0]
    E = layer["n_experts"]
    k = layer["top_k"] if E > 0 else 0
    out = np.empty((T, layer["hidden"]), dtype=np.uint16)
    idx = np.empty((T, max(k, 1)), dtype=np.int32)
    w = np.empty((T, max(k, 1)), dtype=np.float64)
    flag = np.zeros((T,), dtype=np.int32)
    logits = np.empty((T, max(E, 1)), dtype=np.float64)
    fp = None
    if forced_idx is not None:
        fp = np.ascontiguousarray(forced_idx, dtype=np.int32).reshape(T, k)
        keep.append(fp)
    if threads is None:
        threads = host_threads()
    bad = lib().oracle_moe_tokens_mt(ctypes.byref(s), x.ctypes.data, T, _ptr(fp), out.ctypes.data,
                                     idx.ctypes.data, w.ctypes.data, flag.ctypes.data, logits.ctypes.data,
                                     int(threads))
    return dict(out=out, idx=idx[:, :k], w=w[:, :k], flag=flag, logits=logits[:, :E], nan_tokens=int(bad))

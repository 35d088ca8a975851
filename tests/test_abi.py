"""The C-ABI library: it loads, exports every declared symbol, and rejects
bad arguments on the host before touching the GPU (no compute calls here).

Every error case runs twice: through the product entry points of libmoe.so
and through the same checks built alone into libmoe_host.so, a host-only
library that needs no HIP runtime."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "w4a16_routed_expert_sigmoid_amd")
# MOE_HOST_LIB_DIR: the host-only library from another directory (a
# sanitizer build, see test_sanitizers.py).
HOST_LIB = os.path.join(os.environ.get("MOE_HOST_LIB_DIR") or PKG, "libmoe_host.so")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4
W_BF16, W_NVFP4 = 0, 1

# Aligned fake device addresses: validation never dereferences them.
P = 0x7F0000000000
A = lambda i: P + 0x100000 * i  # noqa: E731

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class Desc(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("inter", _i32), ("shared_inter", _i32), ("n_experts", _i32),
                ("top_k", _i32), ("wtype", _i32), ("norm_eps", ctypes.c_float)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("n_q", _i32), ("n_kv", _i32), ("head_dim", _i32), ("window", _i32), ("rope", _i32),
                ("slots", _i32), ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("router_w", "router_b", "w_gate", "w_up", "w_down", "w_scale", "sh_gate", "sh_up",
                                   "sh_down", "sh_scale", "norm_gain")]


def _declare(lib):
    D, W = ctypes.POINTER(Desc), ctypes.POINTER(Weights)
    lib.moe_check_decode_layer.restype = _i32
    lib.moe_check_decode_layer.argtypes = [D, W, _vp, _i32, _vp, _vp, _vp, _vp, _sz]
    lib.moe_check_decode_step.restype = _i32
    lib.moe_check_decode_step.argtypes = [D, W, _i32, _vp, _i32, _vp, _vp, _sz]
    lib.moe_check_prefill_layer.restype = _i32
    lib.moe_check_prefill_layer.argtypes = [D, W, _vp, _i32, _vp, _vp, _vp, _vp, _sz]
    lib.moe_check_repack_nvfp4.restype = _i32
    lib.moe_check_repack_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _i64]
    lib.moe_check_gemv_nvfp4.restype = _i32
    lib.moe_check_gemv_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _vp]
    lib.moe_decode_workspace_bytes.restype = _sz
    lib.moe_decode_workspace_bytes.argtypes = [D, _i32]
    lib.moe_decode_step_workspace_bytes.restype = _sz
    lib.moe_decode_step_workspace_bytes.argtypes = [D, _i32, _i32]
    lib.moe_decode_step_persistent_workspace_bytes.restype = _sz
    lib.moe_decode_step_persistent_workspace_bytes.argtypes = [D, _i32, _i32]
    lib.moe_check_decode_step_persistent.restype = _i32
    lib.moe_check_decode_step_persistent.argtypes = [D, W, _i32, _vp, _i32, _vp, _vp, _sz]
    lib.moe_prefill_workspace_bytes.restype = _sz
    lib.moe_prefill_workspace_bytes.argtypes = [D, _i32]
    lib.moe_nvfp4_matrix_bytes.restype = _sz
    lib.moe_nvfp4_matrix_bytes.argtypes = [_i64, _i64]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [_i32]
    AD = ctypes.POINTER(AttnDesc)
    lib.moe_check_attn_prep.restype = _i32
    lib.moe_check_attn_prep.argtypes = [AD, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.moe_check_attn_decode.restype = _i32
    lib.moe_check_attn_decode.argtypes = [AD, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz]
    lib.moe_check_attn_kv_write.restype = _i32
    lib.moe_check_attn_kv_write.argtypes = [AD, _vp, _vp, _vp, _i32, _i32, _vp, _vp]
    lib.moe_attn_workspace_bytes.restype = _sz
    lib.moe_attn_workspace_bytes.argtypes = [AD, _i32, _i64]
    lib.moe_check_attn_layer.restype = _i32
    lib.moe_check_attn_layer.argtypes = [AD, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]
    return lib


_host = None


def host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            pytest.skip("libmoe_host.so is not built")
        _host = _declare(ctypes.CDLL(HOST_LIB))
    return _host


def hip():
    m = pytest.importorskip("w4a16_routed_expert_sigmoid_amd")
    return m.lib()


LIBS = ["host", "hip"]


def desc(**kw):
    d = dict(hidden=2048, inter=512, shared_inter=512, n_experts=256, top_k=6, wtype=W_NVFP4, norm_eps=1e-6)
    d.update(kw)
    return Desc(**d)


def weights(**kw):
    w = Weights(router_w=A(1), router_b=A(2), w_gate=A(3), w_up=A(4), w_down=A(5), w_scale=A(6),
                sh_gate=A(7), sh_up=A(8), sh_down=A(9), sh_scale=A(10), norm_gain=None)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def decode(which, d=None, w=None, x=A(20), batch=1, y=A(21), idx=None, tw=None, ws=A(22), ws_bytes=1 << 30):
    d, w = d or desc(), w or weights()
    if which == "host":
        return host().moe_check_decode_layer(ctypes.byref(d), ctypes.byref(w), x, batch, y, idx, tw, ws, ws_bytes)
    lib = hip()
    ca = (ctypes.byref(Desc.from_buffer_copy(d)), ctypes.byref(Weights.from_buffer_copy(w)))
    lib.moe_decode_layer.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    return lib.moe_decode_layer(*ca, x, batch, 0, y, idx, tw, ws, ws_bytes, None)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z0-9_]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    m = pytest.importorskip("w4a16_routed_expert_sigmoid_amd")
    names = declared_functions()
    assert "moe_decode_layer" in names and "moe_repack_nvfp4" in names and "moe_prefill_layer" in names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m.EXPORTS)


def test_host_library_needs_no_hip_runtime():
    # It links no HIP library and exports the validation part of the ABI.
    lib = host()
    for n in ("moe_check_decode_layer", "moe_check_decode_step", "moe_check_prefill_layer",
              "moe_check_repack_nvfp4", "moe_decode_workspace_bytes", "moe_decode_step_workspace_bytes",
              "moe_prefill_workspace_bytes", "moe_nvfp4_matrix_bytes", "moe_status_string",
              "moe_check_attn_prep", "moe_check_attn_decode", "moe_attn_workspace_bytes",
              "moe_check_attn_kv_write", "moe_check_attn_layer"):
        assert hasattr(lib, n), n
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert HOST_LIB in maps
    import subprocess
    out = subprocess.run(["ldd", HOST_LIB], capture_output=True, text=True).stdout
    assert "amdhip" not in out and "hsa-runtime" not in out, out


@pytest.mark.parametrize("which", LIBS)
def test_status_strings(which):
    lib = host() if which == "host" else hip()
    lib.moe_status_string.restype = ctypes.c_char_p
    for st in (0, -1, -2, -3, -4):
        s = lib.moe_status_string(st)
        assert s and s != b"unknown status"
    assert lib.moe_status_string(7) == b"unknown status"


def test_matrix_bytes():
    lib = host()
    assert lib.moe_nvfp4_matrix_bytes(512, 2048) == 589824
    assert lib.moe_nvfp4_matrix_bytes(2048, 512) == 589824
    assert lib.moe_nvfp4_matrix_bytes(5632, 2048) == 6488064
    assert lib.moe_nvfp4_matrix_bytes(7, 2048) == 0 and lib.moe_nvfp4_matrix_bytes(8, 48) == 0


def test_workspace_bytes():
    lib = host()
    n1 = lib.moe_decode_workspace_bytes(ctypes.byref(desc()), 1)
    n8 = lib.moe_decode_workspace_bytes(ctypes.byref(desc()), 8)
    n16 = lib.moe_decode_workspace_bytes(ctypes.byref(desc()), 16)
    assert 0 < n1 < n8 < n16
    assert lib.moe_decode_workspace_bytes(ctypes.byref(desc()), 0) == 0
    assert lib.moe_decode_workspace_bytes(ctypes.byref(desc()), 17) == 0
    # BF16 weights: up to 8 tokens
    assert lib.moe_decode_workspace_bytes(ctypes.byref(desc(wtype=W_BF16)), 8) > 0
    assert lib.moe_decode_workspace_bytes(ctypes.byref(desc(wtype=W_BF16)), 9) == 0
    assert lib.moe_decode_workspace_bytes(ctypes.byref(desc(hidden=100)), 1) == 0


TK = A(12)  # room for top-k outputs, clear of the weights, x, y and ws


def test_a_valid_call_passes_validation():
    # The fake buffers are disjoint and large enough: validation says the
    # call would launch (nothing is launched by the check).
    assert decode("host") == OK
    assert decode("host", batch=8, idx=TK, tw=TK + 4096) == OK
    assert decode("host", batch=16, idx=TK, tw=TK + 4096) == OK
    assert prefill("host", idx=TK, tw=TK + 4096) == OK


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(batch=0), INVALID),
    (dict(batch=17), UNSUPPORTED),
    (dict(batch=9, d=desc(wtype=W_BF16)), UNSUPPORTED),                       # BF16 weights: 8 tokens
    (dict(batch=16, d=desc(n_experts=1024, top_k=8)), UNSUPPORTED),          # 17 x 1024 > the routing stage
    (dict(x=None), INVALID),
    (dict(y=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(x=A(20) + 2), INVALID),
    (dict(y=A(20)), INVALID),                          # y == x
    (dict(y=A(20) + 2048), INVALID),                   # y overlaps x (batch 1: 4 KiB each)
    (dict(x=A(22) + 4096), INVALID),                   # x inside the workspace
    (dict(y=A(22) + (1 << 29)), INVALID),              # y inside the workspace
    (dict(idx=A(21) + 16), INVALID),                   # top-k indices overlap y
    (dict(idx=TK, tw=TK + 8), INVALID),                # top-k weights overlap the indices
    (dict(tw=A(22) + 256), INVALID),                   # top-k weights inside the workspace
    (dict(idx=TK + 2), INVALID),                       # misaligned
    (dict(ws=A(22) + 16), INVALID),
    (dict(ws_bytes=100), WORKSPACE),
])
def test_decode_call_errors(which, kw, want):
    assert decode(which, **kw) == want


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(top_k=0), INVALID),
    (dict(top_k=9), INVALID),
    (dict(n_experts=4, top_k=6), INVALID),
    (dict(hidden=2047), INVALID),
    (dict(hidden=0), INVALID),
    (dict(inter=500), INVALID),
    (dict(shared_inter=40), INVALID),
    (dict(wtype=7), INVALID),
    (dict(n_experts=0, shared_inter=0), INVALID),
    (dict(norm_eps=float("nan")), INVALID),
    (dict(n_experts=-1), INVALID),
    (dict(hidden=96), UNSUPPORTED),                    # 3 chunks per row: not tiled
    (dict(inter=32, shared_inter=32), UNSUPPORTED),    # one chunk per row: not tiled
    (dict(inter=96, shared_inter=96), UNSUPPORTED),
    (dict(n_experts=2048), UNSUPPORTED),
    (dict(shared_inter=1024), UNSUPPORTED),            # shared width != routed width
    (dict(hidden=8192), UNSUPPORTED),                  # activations exceed the router's LDS stage at B=8
])
def test_decode_desc_errors(which, kw, want):
    batch = 8 if kw.get("hidden") == 8192 else 1
    assert decode(which, d=desc(**kw), batch=batch) == want


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw", [
    dict(router_w=None), dict(w_gate=None), dict(w_up=None), dict(w_down=None), dict(w_scale=None),
    dict(sh_gate=None), dict(sh_scale=None), dict(w_gate=A(3) + 8), dict(router_b=A(2) + 1),
])
def test_decode_weight_errors(which, kw):
    assert decode(which, w=weights(**kw)) == INVALID


@pytest.mark.parametrize("which", LIBS)
def test_bf16_layer_needs_no_scales(which):
    # BF16 weights with null scale pointers pass validation up to the
    # workspace check (a tiny workspace keeps it off the GPU).
    w = weights(w_scale=None, sh_scale=None)
    assert decode(which, d=desc(wtype=W_BF16), w=w, ws_bytes=1) == WORKSPACE


@pytest.mark.parametrize("which", LIBS)
def test_dense_layer_needs_no_router(which):
    w = weights(router_w=None, w_gate=None, w_up=None, w_down=None, w_scale=None)
    d = desc(n_experts=0, top_k=0, inter=0, shared_inter=5632)
    assert decode(which, d=d, w=w, ws_bytes=1) == WORKSPACE


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("args,want", [
    ((None, A(2), 8, 32, 1), INVALID),
    ((A(1), None, 8, 32, 1), INVALID),
    ((A(1), A(1), 8, 32, 1), INVALID),
    ((A(1), A(1) + 64, 8, 32, 1), INVALID),            # overlapping ranges
    ((A(1), A(2), 7, 32, 1), INVALID),
    ((A(1), A(2), 8, 48, 1), INVALID),
    ((A(1), A(2), 8, 32, 0), INVALID),
    ((A(1) + 4, A(2), 8, 32, 1), INVALID),
])
def test_repack_errors(which, args, want):
    if which == "host":
        assert host().moe_check_repack_nvfp4(*args) == want
        return
    lib = hip()
    assert lib.moe_repack_nvfp4(*args, None, None) == want
    assert lib.moe_unpack_nvfp4(*args, None) == want
    assert lib.moe_dequant_nvfp4(args[0], args[1], *args[2:], None, None) == want


def step(which, dd, ww, n, x, B, y, ws, nbytes):
    if which == "host":
        return host().moe_check_decode_step(dd, ww, n, x, B, y, ws, nbytes)
    lib = hip()
    lib.moe_decode_step.argtypes = [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp]
    return lib.moe_decode_step(ctypes.cast(dd, _vp), ctypes.cast(ww, _vp), n, x, B, y, ws, nbytes, None)


def step_bytes(ds, B):
    arr = (Desc * len(ds))(*ds)
    return host().moe_decode_step_workspace_bytes(arr, len(ds), B)


@pytest.mark.parametrize("which", LIBS)
def test_step_validation(which):
    d = desc()
    dd = (Desc * 2)(d, desc(n_experts=0, top_k=0, inter=0, shared_inter=5632))
    ww = (Weights * 2)(weights(), weights(router_w=None, w_gate=None, w_up=None, w_down=None))
    assert step_bytes([d, dd[1]], 1) > host().moe_decode_workspace_bytes(ctypes.byref(d), 1)
    assert step_bytes([d, desc(hidden=1024)], 1) == 0
    G = 1 << 30
    assert step(which, dd, ww, 0, A(20), 1, A(21), A(22), G) == INVALID
    assert step(which, dd, ww, 2, A(20), 17, A(21), A(22), G) == UNSUPPORTED
    bf = (Desc * 2)(desc(wtype=W_BF16), dd[1])
    assert step(which, bf, ww, 2, A(20), 9, A(21), A(22), G) == UNSUPPORTED
    assert step(which, dd, ww, 2, A(20), 1, A(20), A(22), G) == INVALID
    assert step(which, dd, ww, 2, A(22) + 4096, 1, A(21), A(22), G) == INVALID   # x inside ws
    assert step(which, dd, ww, 2, A(20), 1, A(21), A(22), 64) == WORKSPACE
    bad = (Desc * 2)(d, desc(hidden=1024))
    assert step(which, bad, ww, 2, A(20), 1, A(21), A(22), G) == INVALID
    # a bad weight in the second layer is reported before anything launches
    ww2 = (Weights * 2)(weights(), weights(sh_gate=None))
    assert step(which, dd, ww2, 2, A(20), 1, A(21), A(22), G) == INVALID
    if which == "host":
        assert step(which, dd, ww, 2, A(20), 1, A(21), A(22), G) == OK


def test_step_workspace_covers_every_layer():
    # Layers of different shapes share the step's workspace: the layer part
    # must hold each layer's own workspace (its sync region is laid out for
    # the largest layer), at every batch, and grow with the batch.
    ds = [desc(hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6),
          desc(hidden=256, n_experts=0, top_k=0, inter=0, shared_inter=256),
          desc(hidden=256, inter=128, shared_inter=128, n_experts=64, top_k=8),
          desc(hidden=256, inter=64, shared_inter=0, n_experts=16, top_k=2)]
    lib = host()
    for B in (1, 3, 8):
        s = step_bytes(ds, B)
        act = 2 * ((B * 256 * 2 + 255) // 256 * 256)
        for d in ds:
            assert s - act >= lib.moe_decode_workspace_bytes(ctypes.byref(d), B) > 0
    assert step_bytes(ds, 8) >= step_bytes(ds, 3) >= step_bytes(ds, 1)
    for d in ds:
        assert lib.moe_decode_workspace_bytes(ctypes.byref(d), 8) >= lib.moe_decode_workspace_bytes(ctypes.byref(d), 1)


def prefill(which, d=None, w=None, x=A(20), T=100, y=A(21), idx=None, tw=None, ws=A(22), ws_bytes=1 << 34):
    d, w = d or desc(), w or weights()
    if which == "host":
        return host().moe_check_prefill_layer(ctypes.byref(d), ctypes.byref(w), x, T, y, idx, tw, ws, ws_bytes)
    lib = hip()
    lib.moe_prefill_layer.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    return lib.moe_prefill_layer(ctypes.byref(Desc.from_buffer_copy(d)), ctypes.byref(Weights.from_buffer_copy(w)),
                                 x, T, 0, y, idx, tw, ws, ws_bytes, None)


def test_prefill_workspace_bytes():
    # the expert-sorted rows dominate: (k + 1) * T rows of h [I] and y [H]
    lib = host()
    d = ctypes.byref(desc())
    n = lib.moe_prefill_workspace_bytes(d, 8192)
    assert n >= 7 * 8192 * (512 + 2048) * 2
    assert n < 2 * 7 * 8192 * (512 + 2048) * 2
    assert lib.moe_prefill_workspace_bytes(d, 1) < n
    assert lib.moe_prefill_workspace_bytes(d, 0) == 0
    assert lib.moe_prefill_workspace_bytes(d, (1 << 22) + 1) == 0
    assert lib.moe_prefill_workspace_bytes(ctypes.byref(desc(hidden=100)), 10) == 0


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(T=0), INVALID),
    (dict(T=(1 << 22) + 1), UNSUPPORTED),
    (dict(x=None), INVALID),
    (dict(y=A(20)), INVALID),
    (dict(y=A(20) + 4096), INVALID),                   # y overlaps x (100 tokens: 400 KiB)
    (dict(x=A(22) + (1 << 20)), INVALID),              # x inside the workspace
    (dict(idx=TK, tw=TK + 1024), INVALID),             # weights overlap the indices (2400 B)
    (dict(ws=A(22) + 64), INVALID),
    (dict(x=A(20) + 8), INVALID),
    (dict(ws_bytes=1000), WORKSPACE),
    (dict(d=desc(top_k=9)), INVALID),
    (dict(d=desc(n_experts=2048)), UNSUPPORTED),
    (dict(w=weights(w_down=None)), INVALID),
])
def test_prefill_call_errors(which, kw, want):
    assert prefill(which, **kw) == want


def test_noalloc_rejects_layers_beyond_its_array():
    # The size limit of the no-alloc entry point is checked before any
    # device call: a layer whose batch-8 workspace exceeds the array is
    # refused; validation errors come first.
    m = pytest.importorskip("w4a16_routed_expert_sigmoid_amd")
    lib = m.lib()
    big = desc(hidden=256, inter=4096, shared_inter=4096, n_experts=64, top_k=8)
    assert host().moe_decode_workspace_bytes(ctypes.byref(big), 8) > m.MOE_NOALLOC_SCRATCH_BYTES
    lib.moe_decode_layer_noalloc.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]
    call = lambda d, B: lib.moe_decode_layer_noalloc(ctypes.byref(Desc.from_buffer_copy(d)),  # noqa: E731
                                                     ctypes.byref(Weights.from_buffer_copy(weights())), A(20), B,
                                                     0, A(21), None, None, None)
    assert call(big, 8) == WORKSPACE
    assert call(desc(top_k=9), 1) == INVALID
    assert call(desc(), 17) == UNSUPPORTED
    assert call(desc(), 0) == INVALID


def gemv(which, w=A(1), s=A(2), rows=3072, cols=2048, x=A(20), B=1, y=A(21)):
    if which == "host":
        return host().moe_check_gemv_nvfp4(w, s, rows, cols, x, B, y)
    lib = hip()
    lib.moe_gemv_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp]
    return lib.moe_gemv_nvfp4(w, s, rows, cols, x, B, y, None)


def test_gemv_valid_call_passes_validation():
    assert gemv("host") == OK
    assert gemv("host", w=P + (1 << 36), B=8, rows=131072) == OK   # 151 MB of weights, clear of x and y


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(w=None), INVALID), (dict(s=None), INVALID), (dict(x=None), INVALID), (dict(y=None), INVALID),
    (dict(rows=0), INVALID), (dict(rows=12), INVALID), (dict(cols=48), INVALID), (dict(cols=0), INVALID),
    (dict(B=0), INVALID), (dict(B=9), UNSUPPORTED),
    (dict(cols=96), UNSUPPORTED), (dict(cols=32), UNSUPPORTED), (dict(cols=65536, rows=8), UNSUPPORTED),
    (dict(w=A(1) + 4), INVALID), (dict(x=A(20) + 8), INVALID), (dict(s=A(2) + 2), INVALID),
    (dict(y=A(20)), INVALID),                       # y == x
    (dict(y=A(1) + 4096), INVALID),                 # y inside w (3.5 MB)
    (dict(y=A(2) - 16, B=1, rows=16), INVALID),     # y (32 B) runs over the scale
])
def test_gemv_errors(which, kw, want):
    assert gemv(which, **kw) == want


# ---------------------------------------------------------------- attention

# Caches far apart from everything else (the full-context case is ~1 GB).
KC, VC = P + (1 << 36), P + (2 << 36)


def adesc(**kw):
    d = dict(n_q=32, n_kv=4, head_dim=128, window=513, rope=1, slots=544, rope_theta=10000.0, norm_eps=1e-6)
    d.update(kw)
    return AttnDesc(**d)


def aprep(which, d=None, qkv=A(1), pos=A(2), B=1, qg=A(3), kg=A(4), q=A(5), kc=KC, vc=VC):
    d = d or adesc()
    if which == "host":
        return host().moe_check_attn_prep(ctypes.byref(d), qkv, pos, B, qg, kg, q, kc, vc)
    lib = hip()
    lib.moe_attn_prep.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
    return lib.moe_attn_prep(ctypes.byref(AttnDesc.from_buffer_copy(d)), qkv, pos, B, qg, kg, q, kc, vc, None)


def adecode(which, d=None, q=A(5), kc=KC, vc=VC, pos=A(2), B=1, max_ctx=0, sinks=A(6), out=A(7), ws=A(8),
            ws_bytes=1 << 20):
    d = d or adesc()
    if which == "host":
        return host().moe_check_attn_decode(ctypes.byref(d), q, kc, vc, pos, B, max_ctx, sinks, out, ws, ws_bytes)
    lib = hip()
    lib.moe_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz, _vp]
    return lib.moe_attn_decode(ctypes.byref(AttnDesc.from_buffer_copy(d)), q, kc, vc, pos, B, max_ctx, sinks, out,
                               ws, ws_bytes, None)


def attn_ws(d, B, max_ctx=0):
    return host().moe_attn_workspace_bytes(ctypes.byref(d), B, max_ctx)


def test_attn_valid_calls_pass_validation():
    assert aprep("host") == OK and adecode("host") == OK
    full = adesc(window=0, rope=0, slots=100032)
    assert aprep("host", d=full, B=8) == OK
    assert adecode("host", d=full, B=8, max_ctx=100001, sinks=None, ws_bytes=attn_ws(full, 8, 100001)) == OK


def test_attn_workspace_bytes():
    # one chunk (the 513 window fits in 17 tiles): the status line only
    assert attn_ws(adesc(), 1) == 256 and attn_ws(adesc(), 8) == 256
    # 100,001 positions over 4 KV heads at one token: 64 chunks of 49 tiles;
    # partials of 8 heads x (m, l, 128 values) in FP32
    full = adesc(window=0, rope=0, slots=100032)
    assert attn_ws(full, 1, 100001) == 256 + 64 * 4 * 8 * 130 * 4
    # at 8 tokens: 8 chunks per (token, KV head)
    assert attn_ws(full, 8, 100001) == 256 + 8 * 8 * 4 * 8 * 130 * 4
    # a short context stays in one chunk
    assert attn_ws(full, 1, 700) == 256
    assert attn_ws(full, 1, 100033) == 0 and attn_ws(full, 0, 5) == 0 and attn_ws(adesc(head_dim=64), 1) == 0


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(qkv=None), INVALID), (dict(pos=None), INVALID), (dict(qg=None), INVALID), (dict(kg=None), INVALID),
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vc=None), INVALID),
    (dict(B=0), INVALID), (dict(B=257), INVALID),
    (dict(qkv=A(1) + 8), INVALID), (dict(pos=A(2) + 4), INVALID), (dict(q=A(5) + 2), INVALID),
    (dict(d=adesc(head_dim=64)), UNSUPPORTED), (dict(d=adesc(n_q=64, n_kv=2)), UNSUPPORTED),
    (dict(d=adesc(window=0, slots=(1 << 24) + 32)), UNSUPPORTED),
    (dict(d=adesc(n_q=30)), INVALID), (dict(d=adesc(n_kv=0)), INVALID), (dict(d=adesc(slots=500)), INVALID),
    (dict(d=adesc(window=545)), INVALID), (dict(d=adesc(window=-1)), INVALID), (dict(d=adesc(rope=2)), INVALID),
    (dict(d=adesc(rope_theta=1.0)), INVALID), (dict(d=adesc(norm_eps=-1.0)), INVALID),
    (dict(d=adesc(norm_eps=float("nan"))), INVALID),
    (dict(q=A(1)), INVALID),                 # q_out == qkv
    (dict(q=KC + 4096), INVALID),            # q_out inside the key cache
    (dict(vc=KC + 65536), INVALID),          # the caches overlap
    (dict(kc=A(3)), INVALID),                # the key cache over a gain
])
def test_attn_prep_errors(which, kw, want):
    assert aprep(which, **kw) == want


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vc=None), INVALID), (dict(pos=None), INVALID),
    (dict(out=None), INVALID), (dict(ws=None), INVALID), (dict(B=0), INVALID), (dict(B=257), INVALID),
    (dict(max_ctx=-1), INVALID), (dict(max_ctx=514), INVALID),
    (dict(d=adesc(window=0), max_ctx=545), INVALID),
    (dict(ws=A(8) + 128), INVALID), (dict(sinks=A(6) + 2), INVALID), (dict(out=A(7) + 8), INVALID),
    (dict(d=adesc(head_dim=256)), UNSUPPORTED),
    (dict(out=A(5)), INVALID),               # out == q
    (dict(out=A(6) - 64), INVALID),          # out runs over the sinks
    (dict(ws=KC + 256), INVALID),            # workspace inside the key cache
    (dict(ws_bytes=255), WORKSPACE),
    (dict(d=adesc(window=0, rope=0, slots=100032), max_ctx=100001, ws_bytes=300000), WORKSPACE),
])
def test_attn_decode_errors(which, kw, want):
    assert adecode(which, **kw) == want


def test_attn_sinks_are_optional():
    assert adecode("host", sinks=None) == OK


def akv(which, d=None, k=A(1), v=A(3), pos=A(2), n=100, B=1, kc=KC, vc=VC):
    d = d or adesc()
    if which == "host":
        return host().moe_check_attn_kv_write(ctypes.byref(d), k, v, pos, n, B, kc, vc)
    lib = hip()
    lib.moe_attn_kv_write.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp]
    return lib.moe_attn_kv_write(ctypes.byref(AttnDesc.from_buffer_copy(d)), k, v, pos, n, B, kc, vc, None)


def test_attn_kv_write_valid_call_passes_validation():
    assert akv("host") == OK and akv("host", B=256, n=1) == OK


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(pos=None), INVALID), (dict(kc=None), INVALID),
    (dict(vc=None), INVALID), (dict(n=0), INVALID), (dict(n=(1 << 24) + 1), INVALID), (dict(B=0), INVALID),
    (dict(B=257), INVALID), (dict(k=A(1) + 8), INVALID), (dict(pos=A(2) + 4), INVALID),
    (dict(kc=KC + 2), INVALID), (dict(d=adesc(head_dim=64)), UNSUPPORTED), (dict(d=adesc(slots=40)), INVALID),
    (dict(vc=KC + 4096), INVALID),           # the caches overlap
    (dict(kc=A(3) - 4096), INVALID),         # the key cache runs over the value rows
])
def test_attn_kv_write_errors(which, kw, want):
    assert akv(which, **kw) == want


def test_persistent_step_workspace_and_checks():
    d = desc()
    ds = (Desc * 3)(d, d, d)
    ww = (Weights * 3)(weights(), weights(), weights())
    step = host().moe_decode_step_workspace_bytes(ds, 3, 1)
    pers = host().moe_decode_step_persistent_workspace_bytes(ds, 3, 1)
    # the step's bytes plus 24 per-layer stage sets: logits (16 x 256 FP32),
    # h (16 x 7 x 512 BF16) and the layer input (16 x 2048 BF16)
    assert pers == step + 24 * (16 * 256 * 4 + 16 * 3584 * 2 + 16 * 2048 * 2)
    chk = host().moe_check_decode_step_persistent
    assert chk(ds, ww, 3, A(20), 1, A(21), A(22), pers) == OK
    assert chk(ds, ww, 3, A(20), 1, A(21), A(22), pers - 1) == WORKSPACE
    assert chk(ds, ww, 3, A(20), 17, A(21), A(22), pers) == UNSUPPORTED
    assert chk(ds, ww, 0, A(20), 1, A(21), A(22), pers) == INVALID
    assert chk(ds, ww, 3, A(20), 1, A(20), A(22), pers) == INVALID   # y == x


def alayer(which, d=None, qkv=A(1), pos=A(2), B=1, max_ctx=0, qg=A(3), kg=A(4), sinks=A(6), kc=KC, vc=VC, out=A(7),
           ws=A(8), ws_bytes=1 << 20):
    d = d or adesc()
    if which == "host":
        return host().moe_check_attn_layer(ctypes.byref(d), qkv, pos, B, max_ctx, qg, kg, sinks, kc, vc, out, ws,
                                           ws_bytes)
    lib = hip()
    lib.moe_attn_layer.argtypes = [_vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    return lib.moe_attn_layer(ctypes.byref(AttnDesc.from_buffer_copy(d)), qkv, pos, B, max_ctx, qg, kg, sinks, kc,
                              vc, out, ws, ws_bytes, None)


def test_attn_layer_valid_call_passes_validation():
    assert alayer("host") == OK and alayer("host", sinks=None) == OK
    full = adesc(window=0, rope=0, slots=100032)
    assert alayer("host", d=full, B=8, max_ctx=100001, ws_bytes=attn_ws(full, 8, 100001)) == OK


@pytest.mark.parametrize("which", LIBS)
@pytest.mark.parametrize("kw,want", [
    (dict(qkv=None), INVALID), (dict(pos=None), INVALID), (dict(qg=None), INVALID), (dict(kg=None), INVALID),
    (dict(kc=None), INVALID), (dict(vc=None), INVALID), (dict(out=None), INVALID), (dict(ws=None), INVALID),
    (dict(B=0), INVALID), (dict(B=257), INVALID), (dict(max_ctx=514), INVALID), (dict(ws=A(8) + 16), INVALID),
    (dict(qkv=A(1) + 2), INVALID), (dict(d=adesc(head_dim=64)), UNSUPPORTED),
    (dict(out=A(1)), INVALID),               # out == qkv
    (dict(ws=KC + 4096), INVALID),           # workspace inside the key cache
    (dict(kc=A(3)), INVALID),                # the key cache over a gain
    (dict(ws_bytes=100), WORKSPACE),
])
def test_attn_layer_errors(which, kw, want):
    assert alayer(which, **kw) == want

"""The C-ABI library: it loads, exports every declared symbol, and rejects
bad arguments on the host before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

m = pytest.importorskip("w4a16_routed_expert_sigmoid_amd")

# Aligned fake device addresses: validation never dereferences them.
P = 0x7F0000000000
A = lambda i: P + 0x100000 * i  # noqa: E731


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z0-9_]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "moe_decode_layer" in names and "moe_repack_nvfp4" in names and "moe_prefill_layer" in names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m.EXPORTS)


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert m.status_string(st) and m.status_string(st) != "unknown status"
    assert m.status_string(7) == "unknown status"


def test_matrix_bytes():
    assert m.moe_nvfp4_matrix_bytes(512, 2048) == 589824
    assert m.moe_nvfp4_matrix_bytes(2048, 512) == 589824
    assert m.moe_nvfp4_matrix_bytes(5632, 2048) == 6488064
    assert m.moe_nvfp4_matrix_bytes(7, 2048) == 0 and m.moe_nvfp4_matrix_bytes(8, 48) == 0


def desc(**kw):
    d = dict(hidden=2048, inter=512, shared_inter=512, n_experts=256, top_k=6, wtype=m.MOE_W_NVFP4,
             norm_eps=1e-6)
    d.update(kw)
    return m.moe_layer_desc(**d)


def weights(**kw):
    w = m.moe_layer_weights(router_w=A(1), router_b=A(2), w_gate=A(3), w_up=A(4), w_down=A(5), w_scale=A(6),
                            sh_gate=A(7), sh_up=A(8), sh_down=A(9), sh_scale=A(10), norm_gain=None)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def decode(d=None, w=None, x=A(20), batch=1, y=A(21), ws=A(22), ws_bytes=1 << 30):
    d = d or desc()
    w = w or weights()
    return m.lib().moe_decode_layer(ctypes.byref(d), ctypes.byref(w), x, batch, 0, y, None, None, ws,
                                    ws_bytes, None)


def test_workspace_bytes():
    n1 = m.moe_decode_workspace_bytes(desc(), 1)
    n8 = m.moe_decode_workspace_bytes(desc(), 8)
    assert 0 < n1 < n8
    assert m.moe_decode_workspace_bytes(desc(), 0) == 0
    assert m.moe_decode_workspace_bytes(desc(), 9) == 0
    assert m.moe_decode_workspace_bytes(desc(hidden=100), 1) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(batch=0), m.MOE_ERR_INVALID_ARG),
    (dict(batch=9), m.MOE_ERR_UNSUPPORTED),
    (dict(x=None), m.MOE_ERR_INVALID_ARG),
    (dict(y=None), m.MOE_ERR_INVALID_ARG),
    (dict(ws=None), m.MOE_ERR_INVALID_ARG),
    (dict(x=A(20) + 2), m.MOE_ERR_INVALID_ARG),
    (dict(y=A(20)), m.MOE_ERR_INVALID_ARG),
    (dict(ws=A(22) + 16), m.MOE_ERR_INVALID_ARG),
    (dict(ws_bytes=100), m.MOE_ERR_WORKSPACE),
])
def test_decode_call_errors(kw, want):
    assert decode(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(top_k=0), m.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), m.MOE_ERR_INVALID_ARG),
    (dict(n_experts=4, top_k=6), m.MOE_ERR_INVALID_ARG),
    (dict(hidden=2047), m.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), m.MOE_ERR_INVALID_ARG),
    (dict(inter=500), m.MOE_ERR_INVALID_ARG),
    (dict(shared_inter=40), m.MOE_ERR_INVALID_ARG),
    (dict(wtype=7), m.MOE_ERR_INVALID_ARG),
    (dict(n_experts=0, shared_inter=0), m.MOE_ERR_INVALID_ARG),
    (dict(norm_eps=float("nan")), m.MOE_ERR_INVALID_ARG),
    (dict(n_experts=-1), m.MOE_ERR_INVALID_ARG),
    (dict(hidden=96), m.MOE_ERR_UNSUPPORTED),        # 3 chunks per row: not tiled
    (dict(inter=32, shared_inter=32), m.MOE_ERR_UNSUPPORTED),  # one chunk per row: not tiled
    (dict(inter=96, shared_inter=96), m.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=2048), m.MOE_ERR_UNSUPPORTED),
    (dict(shared_inter=1024), m.MOE_ERR_UNSUPPORTED),  # shared width != routed width
    (dict(hidden=8192), m.MOE_ERR_UNSUPPORTED),        # activations exceed the router's LDS stage at B=8
])
def test_decode_desc_errors(kw, want):
    batch = 8 if kw.get("hidden") == 8192 else 1
    assert decode(d=desc(**kw), batch=batch) == want


@pytest.mark.parametrize("kw", [
    dict(router_w=None), dict(w_gate=None), dict(w_up=None), dict(w_down=None), dict(w_scale=None),
    dict(sh_gate=None), dict(sh_scale=None), dict(w_gate=A(3) + 8), dict(router_b=A(2) + 1),
])
def test_decode_weight_errors(kw):
    assert decode(w=weights(**kw)) == m.MOE_ERR_INVALID_ARG


def test_bf16_layer_needs_no_scales():
    # BF16 weights with null scale pointers pass validation up to the
    # workspace check (a tiny workspace keeps it off the GPU).
    w = weights(w_scale=None, sh_scale=None)
    assert decode(d=desc(wtype=m.MOE_W_BF16), w=w, ws_bytes=1) == m.MOE_ERR_WORKSPACE


def test_dense_layer_needs_no_router():
    w = weights(router_w=None, w_gate=None, w_up=None, w_down=None, w_scale=None)
    d = desc(n_experts=0, top_k=0, inter=0, shared_inter=5632)
    assert decode(d=d, w=w, ws_bytes=1) == m.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("args,want", [
    ((None, A(2), 8, 32, 1), m.MOE_ERR_INVALID_ARG),
    ((A(1), None, 8, 32, 1), m.MOE_ERR_INVALID_ARG),
    ((A(1), A(1), 8, 32, 1), m.MOE_ERR_INVALID_ARG),
    ((A(1), A(1) + 64, 8, 32, 1), m.MOE_ERR_INVALID_ARG),   # overlapping ranges
    ((A(1), A(2), 7, 32, 1), m.MOE_ERR_INVALID_ARG),
    ((A(1), A(2), 8, 48, 1), m.MOE_ERR_INVALID_ARG),
    ((A(1), A(2), 8, 32, 0), m.MOE_ERR_INVALID_ARG),
    ((A(1) + 4, A(2), 8, 32, 1), m.MOE_ERR_INVALID_ARG),
])
def test_repack_errors(args, want):
    lib = m.lib()
    assert lib.moe_repack_nvfp4(*args, None, None) == want
    assert lib.moe_unpack_nvfp4(*args, None) == want
    assert lib.moe_dequant_nvfp4(args[0], args[1], *args[2:], None, None) == want


def test_step_validation():
    lib = m.lib()
    d = desc()
    dd = (m.moe_layer_desc * 2)(d, desc(n_experts=0, top_k=0, inter=0, shared_inter=5632))
    ww = (m.moe_layer_weights * 2)(weights(), weights(router_w=None, w_gate=None, w_up=None, w_down=None))
    assert m.moe_decode_step_workspace_bytes([d, dd[1]], 1) > m.moe_decode_workspace_bytes(d, 1)
    assert m.moe_decode_step_workspace_bytes([d, desc(hidden=1024)], 1) == 0
    assert lib.moe_decode_step(dd, ww, 0, A(20), 1, A(21), A(22), 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_step(dd, ww, 2, A(20), 9, A(21), A(22), 1 << 30, None) == m.MOE_ERR_UNSUPPORTED
    assert lib.moe_decode_step(dd, ww, 2, A(20), 1, A(20), A(22), 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_step(dd, ww, 2, A(20), 1, A(21), A(22), 64, None) == m.MOE_ERR_WORKSPACE
    bad = (m.moe_layer_desc * 2)(d, desc(hidden=1024))
    assert lib.moe_decode_step(bad, ww, 2, A(20), 1, A(21), A(22), 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    # a bad weight in the second layer is reported before anything launches
    ww2 = (m.moe_layer_weights * 2)(weights(), weights(sh_gate=None))
    assert lib.moe_decode_step(dd, ww2, 2, A(20), 1, A(21), A(22), 1 << 30, None) == m.MOE_ERR_INVALID_ARG


def test_step_workspace_covers_every_layer():
    # Layers of different shapes share the step's workspace: the layer part
    # must hold each layer's own workspace (its sync region is laid out for
    # the largest layer), at every batch, and grow with the batch.
    ds = [desc(hidden=256, inter=64, shared_inter=64, n_experts=32, top_k=6),
          desc(hidden=256, n_experts=0, top_k=0, inter=0, shared_inter=256),
          desc(hidden=256, inter=128, shared_inter=128, n_experts=64, top_k=8),
          desc(hidden=256, inter=64, shared_inter=0, n_experts=16, top_k=2)]
    for B in (1, 3, 8):
        step = m.moe_decode_step_workspace_bytes(ds, B)
        act = 2 * ((B * 256 * 2 + 255) // 256 * 256)
        for d in ds:
            assert step - act >= m.moe_decode_workspace_bytes(d, B) > 0
    assert m.moe_decode_step_workspace_bytes(ds, 8) >= m.moe_decode_step_workspace_bytes(ds, 3) >= \
        m.moe_decode_step_workspace_bytes(ds, 1)
    for d in ds:
        assert m.moe_decode_workspace_bytes(d, 8) >= m.moe_decode_workspace_bytes(d, 1)


def prefill(d=None, w=None, x=A(20), T=100, y=A(21), ws=A(22), ws_bytes=1 << 34):
    d = d or desc()
    w = w or weights()
    return m.lib().moe_prefill_layer(ctypes.byref(d), ctypes.byref(w), x, T, 0, y, None, None, ws, ws_bytes,
                                     None)


def test_prefill_workspace_bytes():
    # the expert-sorted rows dominate: (k + 1) * T rows of h [I] and y [H]
    d = desc()
    n = m.moe_prefill_workspace_bytes(d, 8192)
    assert n >= 7 * 8192 * (512 + 2048) * 2
    assert n < 2 * 7 * 8192 * (512 + 2048) * 2
    assert m.moe_prefill_workspace_bytes(d, 1) < n
    assert m.moe_prefill_workspace_bytes(d, 0) == 0
    assert m.moe_prefill_workspace_bytes(d, (1 << 22) + 1) == 0
    assert m.moe_prefill_workspace_bytes(desc(hidden=100), 10) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(T=0), m.MOE_ERR_INVALID_ARG),
    (dict(T=(1 << 22) + 1), m.MOE_ERR_UNSUPPORTED),
    (dict(x=None), m.MOE_ERR_INVALID_ARG),
    (dict(y=A(20)), m.MOE_ERR_INVALID_ARG),
    (dict(ws=A(22) + 64), m.MOE_ERR_INVALID_ARG),
    (dict(x=A(20) + 8), m.MOE_ERR_INVALID_ARG),
    (dict(ws_bytes=1000), m.MOE_ERR_WORKSPACE),
    (dict(d=desc(top_k=9)), m.MOE_ERR_INVALID_ARG),
    (dict(d=desc(n_experts=2048)), m.MOE_ERR_UNSUPPORTED),
    (dict(w=weights(w_down=None)), m.MOE_ERR_INVALID_ARG),
])
def test_prefill_call_errors(kw, want):
    assert prefill(**kw) == want

"""Python binding of libmoe.so, the MI355X small-batch W4A16 sigmoid-routed
MoE layer.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  PyTorch provides device memory and streams.  The entry points
keep the C names (include/moe.h) and take device pointers as integers (or
tensors, whose data_ptr() is used); `stream` defaults to torch's current
stream.  A failing call raises MoeError with the library's status.

The library must have been built (``python w4a16_routed_expert_sigmoid_amd/build.py``
or ``__graft_entry__.build()``); importing fails loudly otherwise.
"""
import ctypes
import os

# PyTorch ships its own HIP runtime.  Load it first so that libmoe.so binds to
# that same runtime instance (matched by soname) instead of a second copy
# from the system ROCm, which would not share devices or memory with torch.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_W_BF16, MOE_W_NVFP4 = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20


class MoeError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        msg = f"{what}: {status_string(status)} ({status})"
        if status == MOE_ERR_HIP:
            msg += ": " + _lib.moe_last_error_detail().decode()
        super().__init__(msg)


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("wtype", ctypes.c_int32),
                ("norm_eps", ctypes.c_float)]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_b", "w_gate", "w_up", "w_down", "w_scale",
        "sh_gate", "sh_up", "sh_down", "sh_scale", "norm_gain")]


class moe_attn_desc(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rope", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_float)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python w4a16_routed_expert_sigmoid_amd/build.py)")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [_i32]
_lib.moe_last_error_detail.restype = ctypes.c_char_p
_lib.moe_last_error_detail.argtypes = []
_lib.moe_nvfp4_matrix_bytes.restype = _sz
_lib.moe_nvfp4_matrix_bytes.argtypes = [_i64, _i64]
_lib.moe_repack_nvfp4.restype = _i32
_lib.moe_repack_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp]
_lib.moe_unpack_nvfp4.restype = _i32
_lib.moe_unpack_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp]
_lib.moe_dequant_nvfp4.restype = _i32
_lib.moe_dequant_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp]
_lib.moe_decode_workspace_bytes.restype = _sz
_lib.moe_decode_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer_desc), _i32]
_lib.moe_decode_layer.restype = _i32
_lib.moe_decode_layer.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _vp,
                                  _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_decode_layer_timed.restype = _i32
_lib.moe_decode_layer_timed.argtypes = _lib.moe_decode_layer.argtypes[:-1] + [ctypes.POINTER(_vp), _vp]
_lib.moe_decode_layer_noalloc.restype = _i32
_lib.moe_decode_layer_noalloc.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _vp,
                                          _i32, _i32, _vp, _vp, _vp, _vp]
_lib.moe_decode_wait_status.restype = _i32
_lib.moe_decode_wait_status.argtypes = [_vp, _vp, _vp]
_lib.moe_decode_step_workspace_bytes.restype = _sz
_lib.moe_decode_step_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer_desc), _i32, _i32]
_lib.moe_decode_step.restype = _i32
_lib.moe_decode_step.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _i32, _vp,
                                 _i32, _vp, _vp, _sz, _vp]
_lib.moe_prefill_workspace_bytes.restype = _sz
_lib.moe_decode_step_persistent_workspace_bytes.restype = _sz
_lib.moe_decode_step_persistent_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer_desc), _i32, _i32]
_lib.moe_decode_step_persistent.restype = _i32
_lib.moe_decode_step_persistent.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _i32,
                                            _vp, _i32, _vp, _vp, _sz, _vp]
_lib.moe_check_decode_step_persistent.restype = _i32
_lib.moe_check_decode_step_persistent.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights),
                                                  _i32, _vp, _i32, _vp, _vp, _sz]
_lib.moe_prefill_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer_desc), _i32]
_lib.moe_prefill_layer.restype = _i32
_lib.moe_prefill_layer.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _vp,
                                   _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]

_lib.moe_gemv_nvfp4.restype = _i32
_lib.moe_gemv_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp]
_lib.moe_check_gemv_nvfp4.restype = _i32
_lib.moe_check_gemv_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _vp]
_lib.moe_probe_hbm_read.restype = _i32
_lib.moe_probe_hbm_read.argtypes = [_vp, _sz, _i32, _vp, _vp]
_lib.moe_check_decode_layer.restype = _i32
_lib.moe_check_decode_layer.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _vp,
                                        _i32, _vp, _vp, _vp, _vp, _sz]
_lib.moe_check_decode_step.restype = _i32
_lib.moe_check_decode_step.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights), _i32,
                                       _vp, _i32, _vp, _vp, _sz]
_lib.moe_check_prefill_layer.restype = _i32
_lib.moe_check_prefill_layer.argtypes = _lib.moe_check_decode_layer.argtypes
_lib.moe_check_repack_nvfp4.restype = _i32
_lib.moe_check_repack_nvfp4.argtypes = [_vp, _vp, _i64, _i64, _i64]

_AD = ctypes.POINTER(moe_attn_desc)
_lib.moe_attn_prep.restype = _i32
_lib.moe_attn_prep.argtypes = [_AD, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.moe_attn_workspace_bytes.restype = _sz
_lib.moe_attn_workspace_bytes.argtypes = [_AD, _i32, _i64]
_lib.moe_attn_decode.restype = _i32
_lib.moe_attn_decode.argtypes = [_AD, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz, _vp]
_lib.moe_check_attn_prep.restype = _i32
_lib.moe_check_attn_prep.argtypes = [_AD, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.moe_attn_kv_write.restype = _i32
_lib.moe_attn_kv_write.argtypes = [_AD, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp]
_lib.moe_check_attn_kv_write.restype = _i32
_lib.moe_check_attn_kv_write.argtypes = [_AD, _vp, _vp, _vp, _i32, _i32, _vp, _vp]
_lib.moe_attn_layer.restype = _i32
_lib.moe_attn_layer.argtypes = [_AD, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_check_attn_layer.restype = _i32
_lib.moe_check_attn_layer.argtypes = [_AD, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]
_lib.moe_check_attn_decode.restype = _i32
_lib.moe_check_attn_decode.argtypes = [_AD, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _sz]

EXPORTS = ("moe_status_string", "moe_last_error_detail", "moe_nvfp4_matrix_bytes", "moe_repack_nvfp4",
           "moe_unpack_nvfp4", "moe_dequant_nvfp4",
           "moe_decode_workspace_bytes", "moe_decode_layer", "moe_decode_layer_timed", "moe_decode_wait_status",
           "moe_decode_layer_noalloc",
           "moe_decode_step_workspace_bytes", "moe_decode_step", "moe_prefill_workspace_bytes",
           "moe_prefill_layer", "moe_check_decode_layer", "moe_check_decode_step", "moe_check_prefill_layer",
           "moe_check_repack_nvfp4", "moe_probe_hbm_read", "moe_gemv_nvfp4", "moe_check_gemv_nvfp4",
           "moe_attn_prep", "moe_attn_workspace_bytes", "moe_attn_decode", "moe_check_attn_prep",
           "moe_check_attn_decode", "moe_attn_kv_write", "moe_check_attn_kv_write",
           "moe_decode_step_persistent", "moe_decode_step_persistent_workspace_bytes",
           "moe_check_decode_step_persistent", "moe_attn_layer", "moe_check_attn_layer")


def lib():
    return _lib


def _ptr(p):
    if p is None:
        return None
    if isinstance(p, int):
        return p
    return p.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st, what):
    if st != MOE_OK:
        raise MoeError(st, what)


def status_string(st):
    return _lib.moe_status_string(st).decode()


def moe_status_string(st):
    return status_string(st)


def moe_last_error_detail():
    return _lib.moe_last_error_detail().decode()


def moe_nvfp4_matrix_bytes(rows, cols):
    return _lib.moe_nvfp4_matrix_bytes(rows, cols)


def moe_repack_nvfp4(src, dst, rows, cols, n_mats, nan_scale_count=None, stream=None):
    _check(_lib.moe_repack_nvfp4(_ptr(src), _ptr(dst), rows, cols, n_mats, _ptr(nan_scale_count),
                                 _stream(stream)), "moe_repack_nvfp4")


def moe_unpack_nvfp4(src, dst, rows, cols, n_mats, stream=None):
    _check(_lib.moe_unpack_nvfp4(_ptr(src), _ptr(dst), rows, cols, n_mats, _stream(stream)),
           "moe_unpack_nvfp4")


def moe_dequant_nvfp4(src, dst, rows, cols, n_mats, tensor_scale=None, stream=None):
    _check(_lib.moe_dequant_nvfp4(_ptr(src), _ptr(dst), rows, cols, n_mats, _ptr(tensor_scale), _stream(stream)),
           "moe_dequant_nvfp4")


def moe_decode_workspace_bytes(desc, max_batch):
    return _lib.moe_decode_workspace_bytes(ctypes.byref(desc), max_batch)


def moe_decode_layer(desc, weights, x, batch, residual, y, topk_idx=None, topk_w=None, ws=None, ws_bytes=0,
                     stream=None):
    _check(_lib.moe_decode_layer(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), batch, int(residual),
                                 _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_decode_layer")


def moe_decode_layer_timed(desc, weights, x, batch, residual, y, topk_idx, topk_w, ws, ws_bytes, events,
                           stream=None):
    """events: 6 torch.cuda.Event (enable_timing=True) attached to the
    layer's kernel dispatches: router, gate/up and down (start, stop)."""
    arr = (_vp * 6)(*[e.cuda_event if hasattr(e, "cuda_event") else e for e in events])
    _check(_lib.moe_decode_layer_timed(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), batch, int(residual),
                                       _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, arr,
                                       _stream(stream)), "moe_decode_layer_timed")


def moe_decode_layer_noalloc(desc, weights, x, batch, residual, y, topk_idx=None, topk_w=None, stream=None):
    """moe_decode_layer with the library's own per-GPU workspace array."""
    _check(_lib.moe_decode_layer_noalloc(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), batch, int(residual),
                                         _ptr(y), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_decode_layer_noalloc")


def moe_decode_wait_status(ws, status_out, stream=None):
    """Enqueue a copy of the workspace's wait status word into status_out
    (a device int32 tensor); ws None: the no-alloc entry point's array."""
    _check(_lib.moe_decode_wait_status(_ptr(ws), _ptr(status_out), _stream(stream)), "moe_decode_wait_status")


def moe_gemv_nvfp4(w, tensor_scale, rows, cols, x, batch, y, stream=None):
    """y[t] = BF16(S * W x[t]) on one repacked NVFP4 matrix, batch 1..8."""
    _check(_lib.moe_gemv_nvfp4(_ptr(w), _ptr(tensor_scale), rows, cols, _ptr(x), batch, _ptr(y), _stream(stream)),
           "moe_gemv_nvfp4")


def moe_attn_prep(desc, qkv, pos, batch, q_gain, k_gain, q_out, k_cache, v_cache, stream=None):
    """Q/K norm + RoPE of `batch` tokens; q to q_out, k and v into the caches."""
    _check(_lib.moe_attn_prep(ctypes.byref(desc), _ptr(qkv), _ptr(pos), batch, _ptr(q_gain), _ptr(k_gain),
                              _ptr(q_out), _ptr(k_cache), _ptr(v_cache), _stream(stream)), "moe_attn_prep")


def moe_attn_layer(desc, qkv, pos, batch, q_gain, k_gain, k_cache, v_cache, out, ws, ws_bytes, max_ctx=0,
                   sinks=None, stream=None):
    """moe_attn_prep + moe_attn_decode in one kernel (no q buffer)."""
    _check(_lib.moe_attn_layer(ctypes.byref(desc), _ptr(qkv), _ptr(pos), batch, max_ctx, _ptr(q_gain), _ptr(k_gain),
                               _ptr(sinks), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(ws), ws_bytes,
                               _stream(stream)), "moe_attn_layer")


def moe_attn_kv_write(desc, k_rows, v_rows, pos, n, batch, k_cache, v_cache, stream=None):
    """K/V rows [batch][n][n_kv][128] into the cache slots of positions pos [batch][n]."""
    _check(_lib.moe_attn_kv_write(ctypes.byref(desc), _ptr(k_rows), _ptr(v_rows), _ptr(pos), n, batch,
                                  _ptr(k_cache), _ptr(v_cache), _stream(stream)), "moe_attn_kv_write")


def moe_attn_workspace_bytes(desc, batch, max_ctx=0):
    return _lib.moe_attn_workspace_bytes(ctypes.byref(desc), batch, max_ctx)


def moe_attn_decode(desc, q, k_cache, v_cache, pos, batch, out, ws, ws_bytes, max_ctx=0, sinks=None,
                    stream=None):
    """Decode attention with sinks and the layer's window over the caches."""
    _check(_lib.moe_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos), batch,
                                max_ctx, _ptr(sinks), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_attn_decode")


def moe_probe_hbm_read(src, nbytes, blocks, sink, stream=None):
    _check(_lib.moe_probe_hbm_read(_ptr(src), nbytes, blocks, _ptr(sink), _stream(stream)), "moe_probe_hbm_read")


def _arrays(descs, weights):
    n = len(descs)
    d = (moe_layer_desc * n)(*descs)
    w = (moe_layer_weights * n)(*weights) if weights is not None else None
    return n, d, w


def moe_decode_step_workspace_bytes(descs, max_batch):
    n, d, _ = _arrays(descs, None)
    return _lib.moe_decode_step_workspace_bytes(d, n, max_batch)


def moe_decode_step(descs, weights, x, batch, y, ws, ws_bytes, stream=None):
    """descs / weights: sequences of moe_layer_desc / moe_layer_weights."""
    n, d, w = _arrays(descs, weights)
    _check(_lib.moe_decode_step(d, w, n, _ptr(x), batch, _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_decode_step")


def moe_decode_step_persistent_workspace_bytes(descs, max_batch):
    n, d, _ = _arrays(descs, None)
    return _lib.moe_decode_step_persistent_workspace_bytes(d, n, max_batch)


def moe_decode_step_persistent(descs, weights, x, batch, y, ws, ws_bytes, stream=None):
    """moe_decode_step with runs of batch-1 MoE layers in one persistent kernel."""
    n, d, w = _arrays(descs, weights)
    _check(_lib.moe_decode_step_persistent(d, w, n, _ptr(x), batch, _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_decode_step_persistent")


def moe_prefill_workspace_bytes(desc, n_tokens):
    return _lib.moe_prefill_workspace_bytes(ctypes.byref(desc), n_tokens)


def moe_prefill_layer(desc, weights, x, n_tokens, residual, y, topk_idx=None, topk_w=None, ws=None,
                      ws_bytes=0, stream=None):
    _check(_lib.moe_prefill_layer(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), n_tokens, int(residual),
                                  _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_prefill_layer")


from .layer import DeviceLayer  # noqa: E402  (device memory holder for one layer)

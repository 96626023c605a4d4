"""ctypes binding of libsf.so: the same entry points as include/sf.h.

Argument marshalling only -- every step of the training path runs in the HIP
library.  Device pointers and streams are passed as integers (for torch:
``tensor.data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``).
Every call raises ``SfError`` on a non-zero status, with the library's
``sf_last_error()`` text.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsf.so")

SF_OK = 0
SF_ERR_ARG = -1
SF_ERR_UNSUPPORTED = -2
SF_ERR_ALIGN = -3
SF_ERR_NOT_PINNED = -4
SF_ERR_POOL = -5
SF_ERR_HIP = -6
SF_ERR_STATE = -7
SF_ERR_NO_DEVICE = -8

SF_F32 = 0
SF_BF16 = 1
SF_F16 = 2

SF_WQ, SF_WK, SF_WV, SF_WO, SF_WG, SF_WU, SF_WD, SF_G1, SF_G2 = range(9)
TENSOR_NAMES = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd", "g1", "g2")

SF_ENGINE_ADAM = 1
SF_ENGINE_HEAD = 2
SF_ENGINE_HEAD_HOST_ADAM = 4
SF_ENGINE_CKPT = 8
SF_ENGINE_PIPELINE = 16
SF_ENGINE_KEEP_TURNAROUND = 32

_size_t = ctypes.c_size_t
_vp = ctypes.c_void_p


class SfShape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32)]


class SfLayout(ctypes.Structure):
    _fields_ = [("off", _size_t * 9), ("bytes", _size_t * 9), ("grad_off", _size_t * 9),
                ("grad_bytes_t", _size_t * 9), ("n_params", _size_t), ("param_bytes", _size_t),
                ("grad_bytes", _size_t), ("saved_bytes", _size_t), ("workspace_bytes", _size_t),
                ("head_workspace_bytes", _size_t)]


class SfEngineCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("window", ctypes.c_int32), ("n_grad_slots", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("adam_threads", ctypes.c_int32), ("lr", ctypes.c_float),
                ("b1", ctypes.c_float), ("b2", ctypes.c_float), ("eps", ctypes.c_float),
                ("d_pool", _vp), ("pool_bytes", _size_t), ("d_act", _vp), ("act_bytes", _size_t),
                ("h_params", ctypes.POINTER(_vp)), ("h_master", ctypes.POINTER(_vp)),
                ("h_m", ctypes.POINTER(_vp)), ("h_v", ctypes.POINTER(_vp)),
                ("h_grad_slots", ctypes.POINTER(_vp)), ("compute_stream", _vp),
                ("d_E", _vp), ("d_gf", _vp), ("d_wlm", _vp), ("d_head_grads", _vp),
                ("h_head_params", _vp), ("h_head_master", _vp), ("h_head_m", _vp), ("h_head_v", _vp),
                ("h_head_grads", _vp), ("d_head_state", _vp), ("h_ckpt", _vp),
                ("loss_scale", ctypes.c_float), ("scale_window", ctypes.c_int32)]


class SfStepStats(ctypes.Structure):
    _fields_ = [("wall_ms", ctypes.c_double), ("compute_ms", ctypes.c_double), ("copy_ms", ctypes.c_double),
                ("h2d_ms", ctypes.c_double), ("d2h_ms", ctypes.c_double), ("overlap_pct", ctypes.c_double),
                ("busy_ms", ctypes.c_double), ("span_ms", ctypes.c_double), ("adam_ms", ctypes.c_double), ("h2d_bytes", ctypes.c_double),
                ("d2h_bytes", ctypes.c_double), ("h2d_gbps", ctypes.c_double), ("d2h_gbps", ctypes.c_double),
                ("loss", ctypes.c_float), ("loss_scale", ctypes.c_float), ("skipped", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class SfError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"sf error {code}: {msg}")
        self.code = code


EXPORTS = (
    "sf_layer_layout", "sf_layer_layout_ex", "sf_ctx_create", "sf_ctx_create_ex", "sf_ctx_destroy", "sf_layer_fwd", "sf_layer_bwd", "sf_head_fwd_bwd",
    "sf_head_fwd_bwd_scaled", "sf_adam_host_ex", "sf_adam_device_ex",
    "sf_gemm", "sf_gemm_workspace_bytes", "sf_gemm_noalloc", "sf_embed_fwd", "sf_embed_bwd", "sf_adam_host", "sf_adam_device", "sf_engine_act_bytes", "sf_engine_act_bytes_flags", "sf_engine_create", "sf_slide_step",
    "sf_engine_sync", "sf_engine_layer_input", "sf_engine_dx0", "sf_engine_trace", "sf_engine_counters",
    "sf_engine_destroy", "sf_last_error",
)

_lib = None


def load():
    """Load libsf.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run layer_sliding_offloaded_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    i32, P = ctypes.c_int32, _vp
    sig = {
        "sf_layer_layout": [ctypes.POINTER(SfShape), i32, ctypes.POINTER(SfLayout)],
        "sf_ctx_create": [ctypes.POINTER(SfShape), i32, P, _size_t, ctypes.POINTER(P)],
        "sf_layer_layout_ex": [ctypes.POINTER(SfShape), i32, i32, ctypes.POINTER(SfLayout)],
        "sf_ctx_create_ex": [ctypes.POINTER(SfShape), i32, i32, P, _size_t, ctypes.POINTER(P)],
        "sf_ctx_destroy": [P],
        "sf_layer_fwd": [P, P, P, P, P, P],
        "sf_layer_bwd": [P, P, P, P, P, P, P, P],
        "sf_head_fwd_bwd": [P, P, P, P, P, P, P, P, P, P],
        "sf_head_fwd_bwd_scaled": [P, P, P, P, P, P, P, P, P, ctypes.c_float, P],
        "sf_adam_host_ex": [i32, P, P, P, P, P, _size_t, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                            ctypes.c_float, ctypes.c_float, ctypes.c_float, i32],
        "sf_adam_device_ex": [i32, P, P, P, P, P, _size_t, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                              ctypes.c_float, ctypes.c_float, ctypes.c_float, P],
        "sf_gemm": [i32, i32, i32, i32, i32, i32, P, ctypes.c_int64, P, ctypes.c_int64, P, ctypes.c_int64,
                    P, _size_t, P],
        "sf_gemm_noalloc": [i32, i32, i32, i32, i32, i32, P, ctypes.c_int64, P, ctypes.c_int64, P,
                            ctypes.c_int64, P],
        "sf_embed_fwd": [P, P, P, P, P],
        "sf_embed_bwd": [P, P, P, P, P],
        "sf_adam_host": [P, P, P, P, P, _size_t, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                         ctypes.c_float, ctypes.c_float, i32],
        "sf_adam_device": [i32, P, P, P, P, P, _size_t, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                           ctypes.c_float, ctypes.c_float, P],
        "sf_engine_act_bytes": [ctypes.POINTER(SfShape), i32, ctypes.POINTER(_size_t)],
        "sf_engine_act_bytes_flags": [ctypes.POINTER(SfShape), i32, i32, ctypes.POINTER(_size_t)],
        "sf_engine_create": [P, ctypes.POINTER(SfEngineCfg), ctypes.POINTER(P)],
        "sf_slide_step": [P, P, P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(SfStepStats)],
        "sf_engine_sync": [P, ctypes.POINTER(SfStepStats)],
        "sf_engine_layer_input": [P, i32, ctypes.POINTER(P)],
        "sf_engine_dx0": [P, ctypes.POINTER(P)],
        "sf_engine_trace": [P, ctypes.POINTER(ctypes.c_double), i32, ctypes.POINTER(i32)],
        "sf_engine_counters": [P, ctypes.POINTER(ctypes.c_int64), i32],
        "sf_engine_destroy": [P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = i32
    lib.sf_gemm_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sf_gemm_workspace_bytes.restype = _size_t
    lib.sf_last_error.argtypes = []
    lib.sf_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def sf_last_error():
    return load().sf_last_error().decode(errors="replace")


def _check(rc):
    if rc != SF_OK:
        raise SfError(rc, sf_last_error())


def make_shape(hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, batch, seq, rms_eps=1e-6, rope_base=10000.0,
               dtype=SF_BF16):
    return SfShape(hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, batch, seq, rms_eps, rope_base, dtype)


def sf_layer_layout(shape, head_chunk_rows=1):
    out = SfLayout()
    _check(load().sf_layer_layout(ctypes.byref(shape), head_chunk_rows, ctypes.byref(out)))
    return out


def sf_layer_layout_ex(shape, head_chunk_rows, head_dw_rows):
    out = SfLayout()
    _check(load().sf_layer_layout_ex(ctypes.byref(shape), head_chunk_rows, head_dw_rows, ctypes.byref(out)))
    return out


def sf_ctx_create(shape, head_chunk_rows, d_workspace, workspace_bytes):
    ctx = _vp()
    _check(load().sf_ctx_create(ctypes.byref(shape), head_chunk_rows, d_workspace, workspace_bytes,
                                ctypes.byref(ctx)))
    return ctx.value


def sf_ctx_create_ex(shape, head_chunk_rows, head_dw_rows, d_workspace, workspace_bytes):
    ctx = _vp()
    _check(load().sf_ctx_create_ex(ctypes.byref(shape), head_chunk_rows, head_dw_rows, d_workspace,
                                   workspace_bytes, ctypes.byref(ctx)))
    return ctx.value


def sf_ctx_destroy(ctx):
    _check(load().sf_ctx_destroy(ctx))


def sf_layer_fwd(ctx, d_w, d_x, d_y, d_saved, stream):
    _check(load().sf_layer_fwd(ctx, d_w, d_x, d_y, d_saved, stream))


def sf_layer_bwd(ctx, d_w, d_x, d_saved, d_dy, d_dx, d_dw, stream):
    _check(load().sf_layer_bwd(ctx, d_w, d_x, d_saved, d_dy, d_dx, d_dw, stream))


def sf_head_fwd_bwd(ctx, d_gf, d_wlm, d_x, d_ids, d_loss, d_dx, d_dgf, d_dwlm, stream):
    _check(load().sf_head_fwd_bwd(ctx, d_gf, d_wlm, d_x, d_ids, d_loss, d_dx, d_dgf, d_dwlm, stream))


def sf_head_fwd_bwd_scaled(ctx, d_gf, d_wlm, d_x, d_ids, d_loss, d_dx, d_dgf, d_dwlm, grad_scale, stream):
    _check(load().sf_head_fwd_bwd_scaled(ctx, d_gf, d_wlm, d_x, d_ids, d_loss, d_dx, d_dgf, d_dwlm, grad_scale,
                                         stream))


def sf_adam_host_ex(dtype, p, m, v, g, p_out, n, step, lr, b1, b2, eps, grad_scale=1.0, n_threads=0):
    """Host pointers (ints); p_out (storage copy) may be None for fp32."""
    _check(load().sf_adam_host_ex(dtype, p, m, v, g, p_out, n, step, lr, b1, b2, eps, grad_scale, n_threads))


def sf_adam_device_ex(dtype, d_p, d_m, d_v, d_g, d_out, n, step, lr, b1, b2, eps, grad_scale, stream):
    _check(load().sf_adam_device_ex(dtype, d_p, d_m, d_v, d_g, d_out, n, step, lr, b1, b2, eps, grad_scale, stream))


def sf_gemm(dtype, layout, out_f32, M, N, K, d_A, lda, d_B, ldb, d_C, ldc, stream, d_ws=None, ws_bytes=0):
    _check(load().sf_gemm(dtype, layout, out_f32, M, N, K, d_A, lda, d_B, ldb, d_C, ldc, d_ws, ws_bytes, stream))


GEMM_STATIC_SCRATCH_BYTES = 64 << 20


def sf_gemm_noalloc(dtype, layout, out_f32, M, N, K, d_A, lda, d_B, ldb, d_C, ldc, stream):
    _check(load().sf_gemm_noalloc(dtype, layout, out_f32, M, N, K, d_A, lda, d_B, ldb, d_C, ldc, stream))


def sf_gemm_workspace_bytes(M, N, K):
    return load().sf_gemm_workspace_bytes(M, N, K)


def sf_embed_fwd(ctx, d_E, d_ids, d_x0, stream):
    _check(load().sf_embed_fwd(ctx, d_E, d_ids, d_x0, stream))


def sf_embed_bwd(ctx, d_dx0, d_ids, d_dE, stream):
    _check(load().sf_embed_bwd(ctx, d_dx0, d_ids, d_dE, stream))


def sf_adam_host(p, m, v, g, p_bf16, n, step, lr, b1, b2, eps, n_threads=0):
    """Host pointers (ints) to fp32 arrays of n elements; p_bf16 may be None."""
    _check(load().sf_adam_host(p, m, v, g, p_bf16, n, step, lr, b1, b2, eps, n_threads))


def sf_adam_device(dtype, d_p, d_m, d_v, d_g, d_out, n, step, lr, b1, b2, eps, stream):
    """Device pointers (ints); d_out (storage-dtype copy) may be None for fp32."""
    _check(load().sf_adam_device(dtype, d_p, d_m, d_v, d_g, d_out, n, step, lr, b1, b2, eps, stream))


def sf_engine_act_bytes(shape, n_layers):
    out = _size_t()
    _check(load().sf_engine_act_bytes(ctypes.byref(shape), n_layers, ctypes.byref(out)))
    return out.value


def sf_engine_act_bytes_flags(shape, n_layers, flags):
    out = _size_t()
    _check(load().sf_engine_act_bytes_flags(ctypes.byref(shape), n_layers, flags, ctypes.byref(out)))
    return out.value


def sf_engine_create(ctx, cfg):
    eng = _vp()
    _check(load().sf_engine_create(ctx, ctypes.byref(cfg), ctypes.byref(eng)))
    return eng.value


def sf_slide_step(eng, d_in, d_dy=None, want_stats=True):
    """Returns (loss, stats) -- loss is None without a head."""
    loss = ctypes.c_float(float("nan"))
    st = SfStepStats()
    _check(load().sf_slide_step(eng, d_in, d_dy, ctypes.byref(loss), ctypes.byref(st) if want_stats else None))
    return loss.value, st


def sf_engine_sync(eng):
    """Drain the engine (pipelined Adam included); returns the measurements of
    the steps since the previous sync."""
    st = SfStepStats()
    _check(load().sf_engine_sync(eng, ctypes.byref(st)))
    return st


def sf_engine_layer_input(eng, layer):
    p = _vp()
    _check(load().sf_engine_layer_input(eng, layer, ctypes.byref(p)))
    return p.value


def sf_engine_dx0(eng):
    p = _vp()
    _check(load().sf_engine_dx0(eng, ctypes.byref(p)))
    return p.value


TRACE_KINDS = {0: "compute", 1: "h2d", 2: "d2h", 3: "adam", 4: "adam_head", 5: "adam_embed"}


def sf_engine_trace(eng):
    """Rows (kind, start_ms, end_ms, info) of the last step's timeline, sorted by start."""
    n = ctypes.c_int32(0)
    _check(load().sf_engine_trace(eng, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_double * (4 * max(1, n.value)))()
    _check(load().sf_engine_trace(eng, buf, n.value, ctypes.byref(n)))
    rows = [tuple(buf[4 * i:4 * i + 4]) for i in range(n.value)]
    return sorted(rows, key=lambda r: (r[1], r[0]))


COUNTER_NAMES = ("events", "events_free", "live_intervals", "window_rows", "blocked_waits")


def sf_engine_counters(eng):
    """The engine's timing bookkeeping as a dict (see COUNTER_NAMES)."""
    buf = (ctypes.c_int64 * len(COUNTER_NAMES))()
    _check(load().sf_engine_counters(eng, buf, len(COUNTER_NAMES)))
    return dict(zip(COUNTER_NAMES, list(buf)))


def sf_engine_destroy(eng):
    _check(load().sf_engine_destroy(eng))


def pointer_array(ptrs):
    """A C array of void* from a list of ints (kept alive by the caller)."""
    arr = (_vp * len(ptrs))(*ptrs)
    return arr

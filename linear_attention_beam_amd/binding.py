"""ctypes binding of libgdnbeam.so: the C ABI of include/gdn_beam.h, same names.

Argument marshalling only.  Every pointer argument accepts an int (device
address), None (NULL), or an object with .data_ptr() (a torch tensor).
Streams accept an int handle, None (the null stream) or an object with
.cuda_stream.  Non-OK statuses raise GdnBeamError.  The library must be built
(python linear_attention_beam_amd/build.py); importing this module without it
raises ImportError, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdnbeam.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_BAD_STATE, GDN_ERR_CAPACITY, GDN_ERR_WORKSPACE, \
    GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = range(7)
GDN_F32, GDN_BF16 = 0, 1
(GDN_EXPORT_ANCESTRY, GDN_EXPORT_TOKENS, GDN_EXPORT_CUM, GDN_EXPORT_GTR_ALPHA,
 GDN_EXPORT_GTR_DELTA, GDN_EXPORT_GTR_KEY, GDN_EXPORT_STATUS) = range(7)

# every entry point the header declares
EXPORTS = ("gdn_beam_workspace_bytes", "gdn_beam_init", "gdn_beam_step", "gdn_beam_select",
           "gdn_beam_export", "gdn_beam_export_bytes", "gdn_beam_query", "gdn_beam_destroy",
           "gdn_beam_status_str", "gdn_beam_last_error", "gdn_beam_prefill",
           "gdn_beam_prefill_workspace_bytes",
           "gdn_fullstate_bytes", "gdn_fullstate_step", "gdn_beam_time_steps", "gdn_beam_step_times",
           "gdn_beam_select_static", "gdn_beam_stamp_projection", "gdn_beam_stream_probe")
GDN_STATIC_SCRATCH_BYTES = 64 << 20


class gdn_beam_config(ctypes.Structure):
    _fields_ = [("R", c_int32), ("H", c_int32), ("d_k", c_int32), ("d_v", c_int32),
                ("T_max", c_int32), ("W_max", c_int32), ("V_max", c_int32),
                ("io_dtype", c_int), ("wout_dtype", c_int), ("H_K", c_int32)]


class GdnBeamError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.gdn_beam_status_str(status).decode()
        if status == GDN_ERR_HIP:
            msg += ": " + _lib.gdn_beam_last_error().decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l and "/" in l})
    except OSError:
        return []


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python linear_attention_beam_amd/build.py")
    # One process must hold one HIP runtime.  PyTorch ships its own copy (same SONAME,
    # different file); loading torch first makes this library bind to that copy.  The
    # other order would map two runtimes that both drive the GPU.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are mapped in this process: {rts}")
    vp, i32, st = c_void_p, c_int32, c_int
    sig = {
        "gdn_beam_workspace_bytes": (st, [POINTER(gdn_beam_config), POINTER(c_size_t)]),
        "gdn_beam_init": (st, [POINTER(gdn_beam_config), vp, i32, vp, c_size_t, vp, POINTER(vp)]),
        "gdn_beam_step": (st, [vp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "gdn_beam_select": (st, [vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]),
        "gdn_beam_select_static": (st, [vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]),
        "gdn_beam_export": (st, [vp, i32, vp, c_size_t, vp]),
        "gdn_beam_export_bytes": (st, [vp, i32, POINTER(c_size_t)]),
        "gdn_beam_query": (st, [vp, POINTER(i32), POINTER(i32)]),
        "gdn_beam_destroy": (None, [vp]),
        "gdn_beam_time_steps": (st, [i32]),
        "gdn_beam_stamp_projection": (st, [vp, c_size_t]),
        "gdn_beam_stream_probe": (st, [vp, vp, c_size_t, i32, vp]),
        "gdn_beam_step_times": (st, [POINTER(ctypes.c_float), i32, POINTER(i32)]),
        "gdn_beam_status_str": (c_char_p, [st]),
        "gdn_beam_last_error": (c_char_p, []),
        "gdn_beam_prefill": (st, [i32, i32, i32, i32, i32, c_int64, vp, vp, vp, vp, vp, vp,
                                  vp, c_size_t, vp]),
        "gdn_beam_prefill_workspace_bytes": (c_size_t, [i32, i32, i32, c_int64]),
        "gdn_fullstate_bytes": (st, [POINTER(gdn_beam_config), POINTER(c_size_t)]),
        "gdn_fullstate_step": (st, [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, c_size_t, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(status: int, where: str):
    if status != GDN_OK:
        raise GdnBeamError(status, where)


def make_config(R, H, d_k, d_v, T_max, W_max, V_max, io="bf16", wout="bf16", H_K=0) -> gdn_beam_config:
    dt = {"f32": GDN_F32, "bf16": GDN_BF16}
    return gdn_beam_config(R, H, d_k, d_v, T_max, W_max, V_max, dt[io], dt[wout], H_K)


def gdn_beam_workspace_bytes(cfg: gdn_beam_config) -> int:
    n = c_size_t(0)
    _check(_lib.gdn_beam_workspace_bytes(byref(cfg), byref(n)), "gdn_beam_workspace_bytes")
    return n.value


def gdn_beam_init(cfg, S_ctx, W0, workspace, workspace_bytes, stream=None) -> int:
    ctx = c_void_p()
    _check(_lib.gdn_beam_init(byref(cfg), _ptr(S_ctx), W0, _ptr(workspace), workspace_bytes,
                              _stream(stream), byref(ctx)), "gdn_beam_init")
    return ctx.value


def gdn_beam_step(ctx, t, q, k, v, alpha, beta, o, stream=None):
    _check(_lib.gdn_beam_step(ctx, t, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                              _ptr(o), _stream(stream)), "gdn_beam_step")


def gdn_beam_select(ctx, t, o, Wout, V, W_next, forced_parent, forced_token, parent, token,
                    score, stream=None):
    _check(_lib.gdn_beam_select(ctx, t, _ptr(o), _ptr(Wout), V, W_next, _ptr(forced_parent),
                                _ptr(forced_token), _ptr(parent), _ptr(token), _ptr(score),
                                _stream(stream)), "gdn_beam_select")


def gdn_beam_select_static(ctx, t, o, Wout, V, W_next, forced_parent, forced_token, parent, token,
                           score, stream=None):
    _check(_lib.gdn_beam_select_static(ctx, t, _ptr(o), _ptr(Wout), V, W_next, _ptr(forced_parent),
                                       _ptr(forced_token), _ptr(parent), _ptr(token), _ptr(score),
                                       _stream(stream)), "gdn_beam_select_static")


def gdn_beam_export_bytes(ctx, what) -> int:
    n = c_size_t(0)
    _check(_lib.gdn_beam_export_bytes(ctx, what, byref(n)), "gdn_beam_export_bytes")
    return n.value


def gdn_beam_export(ctx, what, dst, dst_bytes, stream=None):
    _check(_lib.gdn_beam_export(ctx, what, _ptr(dst), dst_bytes, _stream(stream)), "gdn_beam_export")


def gdn_beam_query(ctx):
    t, w = c_int32(0), c_int32(0)
    _check(_lib.gdn_beam_query(ctx, byref(t), byref(w)), "gdn_beam_query")
    return t.value, w.value


def gdn_beam_destroy(ctx):
    _lib.gdn_beam_destroy(ctx)


def gdn_beam_time_steps(capacity):
    _check(_lib.gdn_beam_time_steps(capacity), "gdn_beam_time_steps")


def gdn_beam_stamp_projection(buf, nbytes):
    _check(_lib.gdn_beam_stamp_projection(_ptr(buf), nbytes), "gdn_beam_stamp_projection")


def gdn_beam_stream_probe(dst, src, nbytes, mode, stream=None):
    _check(_lib.gdn_beam_stream_probe(_ptr(dst), _ptr(src), nbytes, mode, _stream(stream)),
           "gdn_beam_stream_probe")


def gdn_beam_step_times(cap):
    """Durations (ms) of the step launches timed since the last call, in launch order,
    and the number recorded."""
    buf = (ctypes.c_float * max(cap, 1))()
    n = c_int32(0)
    _check(_lib.gdn_beam_step_times(buf, cap, byref(n)), "gdn_beam_step_times")
    return [buf[i] for i in range(min(n.value, cap))], n.value


def gdn_beam_status_str(status: int) -> str:
    return _lib.gdn_beam_status_str(status).decode()


def gdn_beam_last_error() -> str:
    return _lib.gdn_beam_last_error().decode()


def gdn_beam_prefill_workspace_bytes(H, d_k, d_v, N):
    return int(_lib.gdn_beam_prefill_workspace_bytes(H, d_k, d_v, N))


def gdn_beam_prefill(R, H, H_K, d_k, d_v, N, k, v, alpha, beta, offsets, S_out,
                     workspace=None, workspace_bytes=0, stream=None):
    _check(_lib.gdn_beam_prefill(R, H, H_K, d_k, d_v, N, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(offsets), _ptr(S_out), _ptr(workspace), workspace_bytes,
                                 _stream(stream)), "gdn_beam_prefill")


def gdn_fullstate_bytes(cfg: gdn_beam_config) -> int:
    n = c_size_t(0)
    _check(_lib.gdn_fullstate_bytes(byref(cfg), byref(n)), "gdn_fullstate_bytes")
    return n.value


def gdn_fullstate_step(ctx, t, S_ctx, q, k, v, alpha, beta, o, states, states_bytes, stream=None):
    _check(_lib.gdn_fullstate_step(ctx, t, _ptr(S_ctx), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(o), _ptr(states), states_bytes,
                                   _stream(stream)), "gdn_fullstate_step")


def raw_status(name: str, *args) -> int:
    """Call an entry point and return its status code instead of raising (tests)."""
    return getattr(_lib, name)(*args)

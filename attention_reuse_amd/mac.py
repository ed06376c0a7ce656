"""ctypes binding of ``libmac_attention.so`` (argument marshalling only).

Function names follow the C ABI in ``include/mac_attention.h``.  Buffer
arguments accept torch tensors (their ``data_ptr()``), raw integer device
addresses, or None (NULL).  Every compute step runs in the HIP library; this
module raises if the library is missing instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmac_attention.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mac_attention.h")

MAC_OK = 0
MAC_DTYPE_F32 = 0
MAC_DTYPE_BF16 = 1
MAC_THRESH_ONE_MINUS_TAU = 0
MAC_THRESH_TAU = 1
MAC_DEV_BAD_POSITION = 1
MAC_DEV_SYNC_TIMEOUT = 2
MAC_FLAG_FUSED_APPEND = 1
MAC_FLAG_SPLIT_STAGES = 2
MAC_FLAG_SINGLE_LAUNCH = 4
MAC_FLAG_MATCH_FILTER = 8
MAC_FLAG_TWO_STAGES = 16
STATUS = {0: "MAC_OK", -1: "MAC_ERR_INVALID_ARG", -2: "MAC_ERR_UNSUPPORTED",
          -3: "MAC_ERR_HIP", -4: "MAC_ERR_WORKSPACE_TOO_SMALL",
          -5: "MAC_ERR_MISALIGNED", -6: "MAC_ERR_CONTEXT_TOO_LONG",
          -7: "MAC_ERR_NOT_INITIALIZED", -8: "MAC_ERR_SCRATCH_TOO_SMALL"}
MAC_ERR_CONTEXT_TOO_LONG = -6
MAC_ERR_NOT_INITIALIZED = -7
MAC_ERR_SCRATCH_TOO_SMALL = -8
MAC_NOALLOC_SCRATCH_BYTES = 48 << 20
STAGES = ("match", "attend", "merge", "append", "step")


class MacError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(status, "?"), status))
        self.status = status


class mac_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("ring_k", ctypes.c_int32),
        ("band_r", ctypes.c_int32), ("kv_capacity", ctypes.c_int32),
        ("tau", ctypes.c_float), ("thresh_mode", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("flags", ctypes.c_int32),
        ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
        ("kv_stride_t", ctypes.c_int64), ("front_sink", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("max_context", ctypes.c_int32),
        ("min_context", ctypes.c_int32),
    ]


class mac_rings(ctypes.Structure):
    _fields_ = [("q_ring", ctypes.c_void_p), ("o_ring", ctypes.c_void_p),
                ("lse_ring", ctypes.c_void_p), ("pos_ring", ctypes.c_void_p)]


_vp = ctypes.c_void_p
_P = ctypes.POINTER(mac_params)
_R = ctypes.POINTER(mac_rings)
_lib = None


def load():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmac_attention.so is not built (%s); run "
                           "__graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "mac_workspace_bytes": (ctypes.c_size_t, [_P]),
        "mac_ring_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
        "mac_init_rings": (ctypes.c_int, [_P, _R, _vp, ctypes.c_size_t, _vp, _vp,
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                          _vp, _vp, _vp, ctypes.POINTER(_vp)]),
        "mac_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp]),
        "mac_join_aux": (ctypes.c_int, [_vp, _vp]),
        "mac_bind_epochs": (ctypes.c_int, [_vp, _vp]),
        "mac_append_kv": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp, _vp,
                                         _vp]),
        "mac_full_decode": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]),
        "mac_full_decode_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "mac_read_device_status": (ctypes.c_int, [_P, _vp, _vp,
                                                  ctypes.POINTER(ctypes.c_int32)]),
        "mac_profile_start": (ctypes.c_int, [_vp, ctypes.c_int32]),
        "mac_profile_read": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_int32)]),
        "mac_timeline_read": (ctypes.c_int, [_vp, _vp, ctypes.c_size_t]),
        "mac_release": (ctypes.c_int, [_vp]),
        "mac_stream_read": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, ctypes.c_int32, _vp]),
        "mac_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mac_min_chunk_tokens": (ctypes.c_int32, [_P]),
        "mac_chunk_tokens": (ctypes.c_int32, [ctypes.c_int32] * 3),
        "mac_group_items": (ctypes.c_int32, [ctypes.c_int32] * 5 + [
            ctypes.POINTER(ctypes.c_int32)] * 3 + [ctypes.c_int32]),
        "mac_partition": (ctypes.c_int32, [ctypes.c_int32] * 4 + [
            ctypes.POINTER(ctypes.c_int32)] * 2 + [ctypes.c_int32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions declared in the C header."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mac_\w+)\s*\(", text)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(fn, rc):
    if rc != MAC_OK:
        raise MacError(fn, rc)


def make_params(batch, n_q_heads, n_kv_heads, head_dim, kv_dtype, ring_k,
                band_r, kv_capacity, tau, thresh_mode=MAC_THRESH_ONE_MINUS_TAU,
                sm_scale=0.0, strides=(0, 0, 0), flags=0, front_sink=0, page_size=0,
                max_pages=0, page_table=None, max_context=0, min_context=0) -> mac_params:
    """page_table: device tensor or address of the [B, max_pages] int32
    page table when page_size > 0 (the tensor must outlive every call)."""
    return mac_params(batch, n_q_heads, n_kv_heads, head_dim, kv_dtype, ring_k,
                      band_r, kv_capacity, tau, thresh_mode, sm_scale, flags,
                      *strides, front_sink, page_size, max_pages, _ptr(page_table),
                      max_context, min_context)


def mac_workspace_bytes(p: mac_params) -> int:
    return int(load().mac_workspace_bytes(ctypes.byref(p)))


def mac_ring_bytes(p: mac_params):
    out = (ctypes.c_size_t * 4)()
    _check("mac_ring_bytes", load().mac_ring_bytes(ctypes.byref(p), out))
    return tuple(int(x) for x in out)


def mac_init_rings(p: mac_params, q_ring, o_ring, lse_ring, pos_ring, workspace,
                   ws_bytes, warm_qtilde, warm_q, n_warm, ctx_len, k_cache,
                   v_cache, stream=None):
    """Returns the handle (an opaque integer)."""
    rings = mac_rings(_ptr(q_ring), _ptr(o_ring), _ptr(lse_ring), _ptr(pos_ring))
    ctx = (ctypes.c_int32 * p.batch)(*[int(c) for c in ctx_len])
    h = _vp()
    _check("mac_init_rings", load().mac_init_rings(
        ctypes.byref(p), ctypes.byref(rings), _ptr(workspace), int(ws_bytes),
        _ptr(warm_qtilde), _ptr(warm_q), int(n_warm), ctx, _ptr(k_cache),
        _ptr(v_cache), stream, ctypes.byref(h)))
    return h.value


def mac_decode_step(handle, qtilde, q, k_cache, v_cache, pos, out, out_lse=None,
                    match_p=None, match_d2=None, main_stream=None,
                    aux_stream=None):
    _check("mac_decode_step", load().mac_decode_step(
        handle, _ptr(qtilde), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
        _ptr(out), _ptr(out_lse), _ptr(match_p), _ptr(match_d2), main_stream,
        aux_stream))


def mac_append_kv(p: mac_params, k_new, v_new, pos, rope_base, k_cache, v_cache,
                  q_tilde=None, q_out=None, stream=None):
    _check("mac_append_kv", load().mac_append_kv(
        ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(q_tilde), _ptr(q_out), _ptr(pos),
        float(rope_base), _ptr(k_cache), _ptr(v_cache), stream))


def mac_bind_epochs(handle, epoch):
    """Bind a [B] int32 device array of request epochs (None unbinds)."""
    _check("mac_bind_epochs", load().mac_bind_epochs(handle, _ptr(epoch)))


def mac_join_aux(handle, stream=None):
    _check("mac_join_aux", load().mac_join_aux(handle, stream))


def mac_full_decode(p: mac_params, q, k_cache, v_cache, pos, out, out_lse,
                    workspace, ws_bytes, stream=None):
    _check("mac_full_decode", load().mac_full_decode(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
        _ptr(out), _ptr(out_lse), _ptr(workspace), int(ws_bytes), stream))


def mac_full_decode_noalloc(p: mac_params, q, k_cache, v_cache, pos, out, out_lse,
                            stream=None):
    _check("mac_full_decode_noalloc", load().mac_full_decode_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos), _ptr(out),
        _ptr(out_lse), stream))


def mac_read_device_status(p: mac_params, workspace, stream=None) -> int:
    f = ctypes.c_int32()
    _check("mac_read_device_status", load().mac_read_device_status(
        ctypes.byref(p), _ptr(workspace), stream, ctypes.byref(f)))
    return f.value


def mac_profile_start(handle, n_steps):
    _check("mac_profile_start", load().mac_profile_start(handle, int(n_steps)))


def mac_profile_read(handle):
    """Summed milliseconds per stage (dict) and the number of steps."""
    ms = (ctypes.c_double * len(STAGES))()
    n = ctypes.c_int32()
    _check("mac_profile_read", load().mac_profile_read(handle, ms, ctypes.byref(n)))
    return dict(zip(STAGES, list(ms))), n.value


TIMELINE_WGS = 4096
TIMELINE_SLOTS = 32


def mac_timeline_read(handle):
    """The step kernels' timeline words as a list of TIMELINE_WGS lists of
    TIMELINE_SLOTS ints (a library built with MAC_TIMELINE only)."""
    n = TIMELINE_WGS * TIMELINE_SLOTS
    buf = (ctypes.c_uint64 * n)()
    _check("mac_timeline_read", load().mac_timeline_read(handle, buf, ctypes.sizeof(buf)))
    w = list(buf)
    return [w[i * TIMELINE_SLOTS:(i + 1) * TIMELINE_SLOTS] for i in range(TIMELINE_WGS)]


def mac_stream_read(buf, n_bytes, sink, grid, stream=None):
    _check("mac_stream_read", load().mac_stream_read(_ptr(buf), int(n_bytes), _ptr(sink),
                                                     int(grid), stream))


def mac_release(handle):
    _check("mac_release", load().mac_release(handle))


def mac_status_string(status: int) -> str:
    return load().mac_status_string(status).decode()


def mac_min_chunk_tokens(p: mac_params) -> int:
    return int(load().mac_min_chunk_tokens(ctypes.byref(p)))


def mac_chunk_tokens(s: int, e: int, min_chunk: int = 64) -> int:
    return int(load().mac_chunk_tokens(s, e, min_chunk))


def mac_partition(s: int, e: int, r: int, min_chunk: int = 64):
    """[(t0, t1), ...] work items of a KV group attending [s, e] with band r."""
    lib = load()
    n = lib.mac_partition(s, e, r, min_chunk, None, None, 0)
    if n < 0:
        raise ValueError("bad range")
    t0 = (ctypes.c_int32 * n)()
    t1 = (ctypes.c_int32 * n)()
    lib.mac_partition(s, e, r, min_chunk, t0, t1, n)
    return list(zip(t0, t1))


def mac_group_items(s: int, e: int, r: int, front_sink: int, min_chunk: int = 64):
    """([(t0, t1), ...], n_before_split) of a KV group's work items."""
    lib = load()
    n = lib.mac_group_items(s, e, r, front_sink, min_chunk, None, None, None, 0)
    if n < 0:
        raise ValueError("bad range")
    t0 = (ctypes.c_int32 * max(n, 1))()
    t1 = (ctypes.c_int32 * max(n, 1))()
    nb = ctypes.c_int32()
    lib.mac_group_items(s, e, r, front_sink, min_chunk, t0, t1, ctypes.byref(nb), n)
    return list(zip(t0[:n], t1[:n])), nb.value

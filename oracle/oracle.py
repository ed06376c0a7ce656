"""ctypes wrapper over ``mac_oracle.c`` -- TEST INFRASTRUCTURE ONLY.

Arrays are numpy.  K/V and pre-RoPE queries are float32 arrays, or uint16
arrays holding bf16 bit patterns; post-RoPE queries are float32.  All
arithmetic happens in the C file, in fp64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mac_oracle.c")
LIB = os.path.join(HERE, "libmac_oracle.so")
EMPTY_LSE = -math.inf

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)
_lp = ctypes.POINTER(ctypes.c_long)
_vp = ctypes.c_void_p


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int),
        ("ring_k", ctypes.c_int),
        ("band_r", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("ctx_len", ctypes.c_long),
        ("n_warm", ctypes.c_int),
        ("n_steps", ctypes.c_int),
        ("scale", ctypes.c_double),
        ("thresh2", ctypes.c_double),
        ("exempt", ctypes.c_double),
        ("front_sink", ctypes.c_long),
        ("min_context", ctypes.c_long),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libmac_oracle.so``."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=199309L", "-fPIC",
             "-shared", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        lib.mac_oracle_summary.argtypes = [
            ctypes.c_int, _dp, ctypes.c_double, _vp, _vp, ctypes.c_int,
            ctypes.c_long, ctypes.c_long, ctypes.c_long, _dp, _dp]
        lib.mac_oracle_summary.restype = None
        lib.mac_oracle_merge.argtypes = [
            ctypes.c_int, _dp, ctypes.c_double, _dp, ctypes.c_double, _dp, _dp]
        lib.mac_oracle_merge.restype = None
        lib.mac_oracle_rope.argtypes = [ctypes.c_int, _dp, ctypes.c_long, ctypes.c_double,
                                        _dp]
        lib.mac_oracle_rope.restype = None
        lib.mac_oracle_unmerge.argtypes = lib.mac_oracle_merge.argtypes
        lib.mac_oracle_unmerge.restype = None
        lib.mac_oracle_stream.argtypes = [
            ctypes.POINTER(_Cfg), _vp, _vp, ctypes.c_long, _vp, _vp, _vp, _vp,
            _dp, _dp, _ip, _lp, _dp, _dp, _ip, _lp, _dp, _dp, _dp, _dp, _ip]
        lib.mac_oracle_stream.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError("K/V must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _ptr(a, ty=_dp):
    return a.ctypes.data_as(ty) if a is not None else None


def _kv_rows(K: np.ndarray, V: np.ndarray):
    if K.shape != V.shape or K.dtype != V.dtype or K.ndim != 2:
        raise ValueError("K and V must be matching [T, d] arrays")
    if K.strides[1] != K.itemsize or V.strides != K.strides:
        raise ValueError("K/V rows must be contiguous with equal strides")
    return K.strides[0] // K.itemsize


def threshold2(d: int, tau: float, mode: int = 0) -> float:
    """Squared-distance acceptance threshold, computed in fp64 from the fp32
    value of tau and rounded once to fp32.

    mode 0: distance < (1 - tau) * sqrt(2d), i.e. D < 2d (1 - tau)^2 -- the
    blog's worked example (d=128, tau=0.45 gives 8.8) and its pseudocode
    ("MAC-Attention" blog, "Match (2)" and "Paper version").
    mode 1: distance < tau * sqrt(2d), the form given in the paper summary's
    "Core method" section.
    """
    t = float(np.float32(tau))
    f = (1.0 - t) if mode == 0 else t
    return float(np.float32(2.0 * d * f * f))


def summary(q, K, V, a: int, e: int, scale: float | None = None):
    """(o, lse) of query q over positions [a, e] of one KV head."""
    lib = load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    d = q.shape[0]
    rs = _kv_rows(K, V)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros(d, np.float64)
    lse = ctypes.c_double()
    lib.mac_oracle_summary(d, _ptr(q), scale, K.ctypes.data, V.ctypes.data,
                           _dtype_code(K), rs, int(a), int(e), _ptr(o),
                           ctypes.byref(lse))
    return o, lse.value


def rope(x, pos: int, base: float) -> np.ndarray:
    """RoPE of the d-vector x (any float dtype) at position pos, fp64."""
    lib = load()
    x = np.ascontiguousarray(x, np.float64)
    y = np.zeros_like(x)
    lib.mac_oracle_rope(x.shape[0], _ptr(x), int(pos), float(base), _ptr(y))
    return y


def merge(oa, la, ob, lb):
    lib = load()
    oa = np.ascontiguousarray(oa, np.float64)
    ob = np.ascontiguousarray(ob, np.float64)
    o = np.zeros_like(oa)
    lse = ctypes.c_double()
    lib.mac_oracle_merge(oa.shape[0], _ptr(oa), la, _ptr(ob), lb, _ptr(o),
                         ctypes.byref(lse))
    return o, lse.value


def unmerge(ow, lw, op, lp):
    lib = load()
    ow = np.ascontiguousarray(ow, np.float64)
    op = np.ascontiguousarray(op, np.float64)
    o = np.zeros_like(ow)
    lse = ctypes.c_double()
    lib.mac_oracle_unmerge(ow.shape[0], _ptr(ow), lw, _ptr(op), lp, _ptr(o),
                           ctypes.byref(lse))
    return o, lse.value


def run_stream(K, V, qt_warm, q_warm, qt_dec, q_dec, *, ctx_len: int,
               ring_k: int, band_r: int, thresh2: float, n_steps: int | None = None,
               scale: float | None = None, exempt: float = 1e-4,
               want_ring: bool = False, front_sink: int = 0, restart=None,
               min_context: int = 0):
    """Run MAC decode steps for one (request, query head) stream.

    K, V: [T, d] of the head's KV group.  qt_warm: [W, d] pre-RoPE warm
    queries for positions [ctx_len-W, ctx_len-1] (same dtype as K);
    q_warm: [W, d] float32 post-RoPE.  qt_dec / q_dec: [S, d] for decode
    positions ctx_len + s.  front_sink: F leading positions kept out of
    every summary.  restart: optional [S] flags, nonzero where the ring is
    dropped before that step (not ready / invalidated).  min_context:
    positions below it look at no candidate (exact attention, still
    appended).
    """
    lib = load()
    d = K.shape[1]
    rs = _kv_rows(K, V)
    dt = _dtype_code(K)
    qt_warm = np.ascontiguousarray(qt_warm)
    qt_dec = np.ascontiguousarray(qt_dec)
    q_warm = np.ascontiguousarray(q_warm, np.float32)
    q_dec = np.ascontiguousarray(q_dec, np.float32)
    if qt_warm.dtype != K.dtype or qt_dec.dtype != K.dtype:
        raise TypeError("pre-RoPE queries must have the K/V dtype")
    W = qt_warm.shape[0]
    S = qt_dec.shape[0] if n_steps is None else int(n_steps)
    cfg = _Cfg(d, ring_k, band_r, dt, int(ctx_len), W, S,
               (1.0 / math.sqrt(d)) if scale is None else scale,
               float(thresh2), exempt, int(front_sink), int(min_context))
    rst = None
    if restart is not None:
        rst = np.ascontiguousarray(restart, np.int32)
        if rst.shape[0] < S:
            raise ValueError("restart needs one flag per step")
    out = np.zeros((S, d), np.float64)
    lse = np.zeros(S, np.float64)
    hit = np.zeros(S, np.int32)
    p = np.zeros(S, np.int64)
    dist = np.zeros(S, np.float64)
    dist2 = np.zeros(S, np.float64)
    ex = np.zeros(S, np.int32)
    rp = rq = ro = rl = None
    if want_ring:
        rp = np.zeros(ring_k, np.int64)
        rq = np.zeros((ring_k, d), np.float64)
        ro = np.zeros((ring_k, d), np.float64)
        rl = np.zeros(ring_k, np.float64)
    ws = ctypes.c_double()
    rc = lib.mac_oracle_stream(
        ctypes.byref(cfg), K.ctypes.data, V.ctypes.data, rs,
        qt_warm.ctypes.data, q_warm.ctypes.data, qt_dec.ctypes.data,
        q_dec.ctypes.data, _ptr(out), _ptr(lse), _ptr(hit, _ip), _ptr(p, _lp),
        _ptr(dist), _ptr(dist2), _ptr(ex, _ip), _ptr(rp, _lp), _ptr(rq),
        _ptr(ro), _ptr(rl), ctypes.byref(ws), _ptr(rst, _ip))
    if rc != 0:
        raise MemoryError("oracle stream allocation failed")
    res = dict(out=out, lse=lse, hit=hit.astype(bool), p=p, dist=dist,
               dist2=dist2, exempt=ex.astype(bool), warm_seconds=ws.value)
    if want_ring:
        res.update(ring_pos=rp, ring_q=rq, ring_o=ro, ring_lse=rl)
    return res


def run_streams(K, V, qt, q, heads, *, ctx_len: int, n_warm: int, ring_k: int,
                band_r: int, thresh2: float, n_steps: int | None = None,
                threads: int | None = None, want_ring: bool = False,
                front_sink: int = 0, restart=None, min_context: int = 0):
    """Run many (b, h) streams in parallel threads (ctypes drops the GIL).

    K, V: [B, Hkv, T, d]; qt, q: [B, Hq, W+S, d] (warm part first).
    heads: iterable of (b, h).  restart: optional [B, S] flags (see
    run_stream).  Returns {(b, h): result}.
    """
    Hq, Hkv = qt.shape[1], K.shape[1]
    G = Hq // Hkv
    W = n_warm

    def one(bh):
        b, h = bh
        g = h // G
        return bh, run_stream(
            K[b, g], V[b, g], qt[b, h, :W], q[b, h, :W], qt[b, h, W:],
            q[b, h, W:], ctx_len=ctx_len, ring_k=ring_k, band_r=band_r,
            thresh2=thresh2, n_steps=n_steps, want_ring=want_ring,
            front_sink=front_sink, restart=None if restart is None else restart[b],
            min_context=min_context)

    heads = list(heads)
    nt = threads or min(len(heads), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=max(1, nt)) as ex:
        return dict(ex.map(one, heads))


def full_decode(q, K, V, m, scale: float | None = None):
    """Full attention for every (b, h): q [B, Hq, d] float32, K/V
    [B, Hkv, T, d], m [B] last attended position.  Returns (out, lse)."""
    B, Hq, d = q.shape
    G = Hq // K.shape[1]
    out = np.zeros((B, Hq, d), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h], lse[b, h] = summary(q[b, h], K[b, h // G], V[b, h // G],
                                           0, int(m[b]), scale)
    return out, lse

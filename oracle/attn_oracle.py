"""ctypes front end of the fp64 C oracle -- TEST INFRASTRUCTURE ONLY.

Follows the attention fixture of the LuisaCompute "Attention execution
mapping" review (section 1): bottom-right causal GQA, kv-head h/(Hq/Hkv),
legal keys k <= q + K_b - Q (K_b replaces K for per-sequence lengths), an
optional window of W keys ending at the diagonal, O = 0 / LSE = -inf for rows
without a legal key; with causal=False every key k < K_b is legal for every
row (no window).  Inputs are host arrays: bf16 as uint16 bit patterns,
float32, IEEE binary16 (numpy float16) or float64 (for finite-difference
checks).  Results are float64.  `bwd` gives the gradients of sum(dO * O)
with respect to q, k and v.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_libs: dict[str, ctypes.CDLL] = {}


def _setup(lib):
    vp, ci, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_attn_fwd.argtypes = [vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, dbl,
                                    i64, i64, i64, i64, ci, ci]
    lib.oracle_attn_fwd.restype = ci
    lib.oracle_attn_fwd_rows.argtypes = [vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, dbl,
                                         vp, i64, ci, ci]
    lib.oracle_attn_fwd_rows.restype = ci
    lib.oracle_attn_probs.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, dbl, ci, ci, ci, vp, ci]
    lib.oracle_attn_probs.restype = i64
    lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, ci, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, dbl, ci, ci]
    lib.oracle_attn_bwd.restype = ci
    lib.oracle_attn_bwd_rows.argtypes = [vp, vp, vp, vp, ci, vp, i64, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, dbl, ci,
                                         ci]
    lib.oracle_attn_bwd_rows.restype = ci
    lib.oracle_attn_bwd_keys.argtypes = [vp, vp, vp, vp, ci, vp, i64, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, dbl,
                                         ci, ci]
    lib.oracle_attn_bwd_keys.restype = ci
    return lib


def load(path: str | None = None) -> "Oracle":
    path = path or _build.LIB
    if path == _build.LIB and not os.path.exists(path):
        _build.build()
    if path not in _libs:
        _libs[path] = _setup(ctypes.CDLL(path))
    return Oracle(_libs[path])


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.uint16:
        return 0
    if arr.dtype == np.float32:
        return 1
    if arr.dtype == np.float16:
        return 2
    if arr.dtype == np.float64:
        return 3
    raise TypeError("oracle inputs are bf16 bit patterns (uint16), float32, float16 or float64")


def _threads(threads: int) -> int:
    if threads and threads > 0:
        return threads
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class OracleError(RuntimeError):
    pass


class Oracle:
    def __init__(self, lib):
        self.lib = lib

    def fwd(self, q, k, v, *, seqlens=None, window=0, scale=None, threads=0, ld=None, causal=True):
        """Full forward.  q [B,Hq,Q,*], k [B,Hkv,K,*], v [B,Hkv,K,*] (row strides taken
        from the last axis unless `ld` = (ldq, ldk, ldv, ldo, D, Dv) is given).
        Returns (o [B,Hq,Q,Dv] float64, lse [B,Hq,Q] float64)."""
        B, Hq, Q, ldq = q.shape
        _, Hkv, K, ldk = k.shape
        ldv = v.shape[-1]
        if ld is None:
            D, Dv, ldo = ldq, ldv, ldv
        else:
            ldq, ldk, ldv, ldo, D, Dv = ld
        code = _dtype_code(q)
        assert _dtype_code(k) == code and _dtype_code(v) == code
        for a in (q, k, v):
            assert a.flags.c_contiguous
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        o = np.empty((B, Hq, Q, ldo), dtype=np.float64)
        lse = np.empty((B, Hq, Q), dtype=np.float64)
        sl = None
        if seqlens is not None:
            sl = np.ascontiguousarray(seqlens, dtype=np.int32)
        rc = self.lib.oracle_attn_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, code, o.ctypes.data,
                                      lse.ctypes.data, B, Hq, Hkv, Q, K, D, Dv,
                                      None if sl is None else sl.ctypes.data, int(window), float(scale),
                                      ldq, ldk, ldv, ldo, _threads(threads), int(bool(causal)))
        if rc:
            raise OracleError(f"oracle_attn_fwd returned {rc}")
        return o, lse

    def fwd_into(self, q, k, v, o, lse, *, D, Dv, seqlens=None, window=0, scale=None, threads=0, causal=True):
        """Like fwd but writes into caller-provided wide rows (o's last axis may exceed Dv)."""
        B, Hq, Q, ldq = q.shape
        _, Hkv, K, ldk = k.shape
        ldv, ldo = v.shape[-1], o.shape[-1]
        assert o.dtype == np.float64 and o.flags.c_contiguous and lse.dtype == np.float64
        code = _dtype_code(q)
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        rc = self.lib.oracle_attn_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, code, o.ctypes.data,
                                      lse.ctypes.data, B, Hq, Hkv, Q, K, D, Dv,
                                      None if sl is None else sl.ctypes.data, int(window), float(scale),
                                      ldq, ldk, ldv, ldo, _threads(threads), int(bool(causal)))
        if rc:
            raise OracleError(f"oracle_attn_fwd returned {rc}")

    def rows(self, q, k, v, rows, *, seqlens=None, window=0, scale=None, threads=0, shape=None, causal=True):
        """Selected flat rows (b*Hq+h)*Q+q.  q/k/v may be full arrays, or any buffers when
        `shape` = (B,Hq,Hkv,Q,K,D,Dv) is given.  Returns (o [n,Dv], lse [n])."""
        if shape is None:
            B, Hq, Q, D = q.shape
            _, Hkv, K, _ = k.shape
            Dv = v.shape[-1]
        else:
            B, Hq, Hkv, Q, K, D, Dv = shape
        code = _dtype_code(q)
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((len(r), Dv), dtype=np.float64)
        lse = np.empty((len(r),), dtype=np.float64)
        sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        rc = self.lib.oracle_attn_fwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, code, o.ctypes.data,
                                           lse.ctypes.data, B, Hq, Hkv, Q, K, D, Dv,
                                           None if sl is None else sl.ctypes.data, int(window), float(scale),
                                           r.ctypes.data, len(r), _threads(threads), int(bool(causal)))
        if rc:
            raise OracleError(f"oracle_attn_fwd_rows returned {rc}")
        return o, lse

    def probs(self, q, k, b, h, qi, *, seqlens=None, window=0, scale=None, causal=True):
        """Normalised weights of one row over all K key slots (0 where not legal)."""
        B, Hq, Q, D = q.shape
        _, Hkv, K, _ = k.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        p = np.empty((max(K, 1),), dtype=np.float64)
        sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        n = self.lib.oracle_attn_probs(q.ctypes.data, k.ctypes.data, _dtype_code(q), B, Hq, Hkv, Q, K, D,
                                       None if sl is None else sl.ctypes.data, int(window), float(scale),
                                       b, h, qi, p.ctypes.data, int(bool(causal)))
        if n < 0:
            raise OracleError(f"oracle_attn_probs returned {n}")
        return p[:K], int(n)

    def bwd(self, q, k, v, dout, *, seqlens=None, window=0, scale=None, threads=0, causal=True):
        """Gradients of sum(dout * O) w.r.t. q, k, v (dense [B,H,T,width] inputs, dout
        [B,Hq,Q,Dv] in the same dtype).  Returns (dq, dk, dv) float64."""
        B, Hq, Q, D = q.shape
        _, Hkv, K, _ = k.shape
        Dv = v.shape[-1]
        code = _dtype_code(q)
        for a in (k, v, dout):
            assert _dtype_code(a) == code
        for a in (q, k, v, dout):
            assert a.flags.c_contiguous
        assert dout.shape == (B, Hq, Q, Dv)
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        dq = np.empty((B, Hq, Q, D), dtype=np.float64)
        dk = np.empty((B, Hkv, K, D), dtype=np.float64)
        dv = np.empty((B, Hkv, K, Dv), dtype=np.float64)
        sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        rc = self.lib.oracle_attn_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, code,
                                      dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, B, Hq, Hkv, Q, K, D, Dv,
                                      None if sl is None else sl.ctypes.data, int(window), float(scale),
                                      _threads(threads), int(bool(causal)))
        if rc:
            raise OracleError(f"oracle_attn_bwd returned {rc}")
        return dq, dk, dv

    def bwd_rows(self, q, k, v, dout, rows, *, seqlens=None, window=0, scale=None, threads=0, causal=True):
        """dq of selected flat rows (b*Hq+h)*Q+q.  Returns [n, D] float64."""
        B, Hq, Q, D = q.shape
        _, Hkv, K, _ = k.shape
        Dv = v.shape[-1]
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((len(r), D), dtype=np.float64)
        sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        rc = self.lib.oracle_attn_bwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                           _dtype_code(q), r.ctypes.data, len(r), out.ctypes.data, B, Hq, Hkv, Q, K,
                                           D, Dv, None if sl is None else sl.ctypes.data, int(window), float(scale),
                                           _threads(threads), int(bool(causal)))
        if rc:
            raise OracleError(f"oracle_attn_bwd_rows returned {rc}")
        return out

    def bwd_keys(self, q, k, v, dout, keys, *, seqlens=None, window=0, scale=None, threads=0, causal=True):
        """dk, dv of selected flat keys (b*Hkv+kh)*K+k.  Returns ([n, D], [n, Dv]) float64."""
        B, Hq, Q, D = q.shape
        _, Hkv, K, _ = k.shape
        Dv = v.shape[-1]
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        kk = np.ascontiguousarray(keys, dtype=np.int64)
        dk = np.empty((len(kk), D), dtype=np.float64)
        dv = np.empty((len(kk), Dv), dtype=np.float64)
        sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        rc = self.lib.oracle_attn_bwd_keys(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                           _dtype_code(q), kk.ctypes.data, len(kk), dk.ctypes.data, dv.ctypes.data, B,
                                           Hq, Hkv, Q, K, D, Dv, None if sl is None else sl.ctypes.data, int(window),
                                           float(scale), _threads(threads), int(bool(causal)))
        if rc:
            raise OracleError(f"oracle_attn_bwd_keys returned {rc}")
        return dk, dv

"""Seeded synthetic inputs for the causal GQA attention forward.

This module generates host arrays only: Q/K/V as iid N(0,1) rounded to bf16
(or kept fp32), and int32 per-sequence KV lengths.  It holds none of the
attention arithmetic, so the GPU path and the CPU oracle can both consume its
output without sharing any code of the method.

Streams are Philox-4x32-10 keyed by (seed, tensor_id) with tensor ids
Q=1, K=2, V=3, seqlens=4, so any slice of any tensor can be regenerated on its
own from its flat element offset (the parity tests use this to check sampled
rows of multi-GiB workloads without materialising them twice).

The seed of the test protocol on the Laya "Fast backends" page (section
"Numerics") is 1234; bf16 inputs are rounded once and both sides read the same
rounded values.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED = 1234
TID_Q, TID_K, TID_V, TID_SEQLENS = 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn_inputs.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build_inputs()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, u32, vp, ci = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
        lib.attn_inputs_normal_bf16.argtypes = [vp, i64, i64, u32, u32, ci]
        lib.attn_inputs_normal_f32.argtypes = [vp, i64, i64, u32, u32, ci]
        lib.attn_inputs_u32.argtypes = [vp, i64, i64, u32, u32]
        lib.attn_inputs_philox4x32_10.argtypes = [vp, vp, vp]
        lib.attn_inputs_f32_to_bf16.argtypes = [vp, vp, i64]
        for f in (lib.attn_inputs_normal_bf16, lib.attn_inputs_normal_f32, lib.attn_inputs_u32,
                  lib.attn_inputs_philox4x32_10, lib.attn_inputs_f32_to_bf16):
            f.restype = None
        _lib = lib
    return _lib


def host_threads() -> int:
    """Threads this process may run on (affinity-aware)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def philox4x32_10(ctr, key) -> list[int]:
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.attn_inputs_philox4x32_10(c, k, o)
    return list(o)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().attn_inputs_f32_to_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, tensor_id: int, seed: int = SEED, dtype: str = "bf16", offset: int = 0,
           threads: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """N(0,1) samples for elements [offset, offset+prod(shape)) of stream (seed, tensor_id).

    dtype "bf16" returns the uint16 bit patterns; "f32" returns float32; "f16"
    returns float16, the float32 stream rounded to nearest even (numpy's
    conversion).
    """
    n = int(np.prod(shape)) if len(shape) else 1
    lib = _load()
    if dtype == "bf16":
        arr = out if out is not None else np.empty(shape, dtype=np.uint16)
        assert arr.dtype == np.uint16 and arr.size == n and arr.flags.c_contiguous
        lib.attn_inputs_normal_bf16(arr.ctypes.data, n, offset, seed, tensor_id, threads or host_threads())
    elif dtype == "f32":
        arr = out if out is not None else np.empty(shape, dtype=np.float32)
        assert arr.dtype == np.float32 and arr.size == n and arr.flags.c_contiguous
        lib.attn_inputs_normal_f32(arr.ctypes.data, n, offset, seed, tensor_id, threads or host_threads())
    elif dtype == "f16":
        tmp = np.empty(shape, dtype=np.float32)
        lib.attn_inputs_normal_f32(tmp.ctypes.data, n, offset, seed, tensor_id, threads or host_threads())
        arr = out if out is not None else np.empty(shape, dtype=np.float16)
        assert arr.dtype == np.float16 and arr.size == n and arr.flags.c_contiguous
        arr[...] = tmp.astype(np.float16)
    else:
        raise ValueError(f"dtype must be 'bf16', 'f16' or 'f32', got {dtype!r}")
    return arr


def uniform_words(n: int, tensor_id: int, seed: int = SEED, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    _load().attn_inputs_u32(out.ctypes.data, n, offset, seed, tensor_id)
    return out


def _unit(words: np.ndarray) -> np.ndarray:
    """Map 32-bit words to doubles in (0,1)."""
    return (words.astype(np.float64) + 0.5) / 4294967296.0


def seqlens_uniform(B: int, kmax: int, zero_at=(), seed: int = SEED) -> np.ndarray:
    """int32 lengths uniform on [0, kmax]: floor(u*(kmax+1)); listed indices forced to 0."""
    u = _unit(uniform_words(B, TID_SEQLENS, seed))
    s = np.minimum(np.floor(u * (kmax + 1)), kmax).astype(np.int32)
    for b in zero_at:
        s[b] = 0
    return s


def seqlens_loguniform(B: int, lo: int, hi: int, seed: int = SEED) -> np.ndarray:
    """int32 lengths log-uniform on [lo, hi]: min(hi, floor(lo*(hi/lo)^u))."""
    u = _unit(uniform_words(B, TID_SEQLENS, seed))
    s = np.floor(lo * np.power(hi / lo, u))
    return np.clip(s, lo, hi).astype(np.int32)


@dataclass
class Workload:
    """One attention-forward problem: shapes, options and the recipe of its inputs."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Q: int
    K: int
    D: int
    Dv: int
    dtype: str = "bf16"          # "bf16" (bf16 in, bf16 O), "f16" (fp16 in, fp16 O) or "f32"
    window: int = 0              # <= 0: no sliding window
    seqlens: Optional[np.ndarray] = None   # int32[B] or None (every K_b = K)
    seed: int = SEED
    note: str = ""
    scale: Optional[float] = None
    causal: bool = True          # False: every key k < K_b is legal for every row (no window)

    def __post_init__(self):
        if self.scale is None:
            self.scale = 1.0 / math.sqrt(self.D)

    @property
    def shape_tuple(self):
        return (self.B, self.Hq, self.Hkv, self.Q, self.K, self.D, self.Dv)

    def q_shape(self):
        return (self.B, self.Hq, self.Q, self.D)

    def k_shape(self):
        return (self.B, self.Hkv, self.K, self.D)

    def v_shape(self):
        return (self.B, self.Hkv, self.K, self.Dv)

    def o_shape(self):
        return (self.B, self.Hq, self.Q, self.Dv)

    def kb(self, b: int) -> int:
        return int(self.seqlens[b]) if self.seqlens is not None else self.K

    def legal_pairs(self) -> int:
        """Number of (row, key) pairs the causal/window/length predicate admits (host count)."""
        total = 0
        for b in range(self.B):
            Kb = self.kb(b)
            if not self.causal:
                total += self.Q * Kb
                continue
            for q in range(self.Q):
                p = q + Kb - self.Q
                hi = min(Kb - 1, p)
                lo = 0 if self.window <= 0 else max(0, p - self.window + 1)
                if hi >= lo:
                    total += hi - lo + 1
        return total * self.Hq

    def kv_tokens(self) -> int:
        """Sum over sequences of K_b times kv-heads: the KV rows a single-pass kernel must read."""
        return self.Hkv * sum(self.kb(b) for b in range(self.B))

    def gen_q(self, threads: int = 0):
        return normal(self.q_shape(), TID_Q, self.seed, self.dtype, threads=threads)

    def gen_k(self, threads: int = 0, padding: str = "normal"):
        return self._gen_kv(self.k_shape(), TID_K, threads, padding)

    def gen_v(self, threads: int = 0, padding: str = "normal"):
        return self._gen_kv(self.v_shape(), TID_V, threads, padding)

    def _gen_kv(self, shape, tid, threads, padding):
        """K or V.  padding="normal" fills every row from the stream; "zero" fills
        only rows k < K_b (same values as "normal" there) and leaves the padding
        rows zero, which the attention never reads, to save generation time on
        long padded caches."""
        if padding == "normal" or self.seqlens is None:
            return normal(shape, tid, self.seed, self.dtype, threads=threads)
        if padding != "zero":
            raise ValueError(f"padding must be 'normal' or 'zero', got {padding!r}")
        arr = np.zeros(shape, dtype={"bf16": np.uint16, "f16": np.float16, "f32": np.float32}[self.dtype])
        B, H, T, W = shape
        for b in range(B):
            kb = self.kb(b)
            for hh in range(H):
                if kb > 0:
                    normal((kb, W), tid, self.seed, self.dtype, offset=((b * H + hh) * T) * W,
                           threads=threads, out=arr[b, hh, :kb])
        return arr

    def gen_rows(self, which: str, b: int, head: int, r0: int, r1: int) -> np.ndarray:
        """Regenerate rows [r0, r1) of one (batch, head) slice of Q, K or V on its own."""
        shp = {"q": self.q_shape(), "k": self.k_shape(), "v": self.v_shape()}[which]
        tid = {"q": TID_Q, "k": TID_K, "v": TID_V}[which]
        _, H, T, W = shp
        off = ((b * H + head) * T + r0) * W
        return normal((r1 - r0, W), tid, self.seed, self.dtype, offset=off)


def config(idx: int) -> Workload:
    """The five benchmark workloads, 1-based, in the order the metric lists them."""
    if idx == 1:
        return Workload("c1_tiny_fp32_prefill", 1, 4, 2, 64, 128, 64, 64, dtype="f32",
                        note="tiny fp32 bottom-right causal GQA, contiguous [B,H,T,D]")
    if idx == 2:
        return Workload("c2_decode_tail_2053", 1, 8, 2, 1, 2053, 80, 96,
                        note="single-sequence decode, K tail 2053 = 32*64+5, D != Dv")
    if idx == 3:
        return Workload("c3_dense_causal_prefill", 4, 32, 8, 4096, 4096, 128, 128,
                        note="dense causal GQA prefill, Q = K = 4096")
    if idx == 4:
        return Workload("c4_varlen_window_prefill", 16, 32, 8, 4096, 4096, 128, 128, window=1024,
                        seqlens=seqlens_uniform(16, 4096, zero_at=(1, 14)),
                        note="varlen padded prefill, seqlens uniform [0,4096], b=1 and b=14 forced to 0, window 1024")
    if idx == 5:
        return Workload("c5_batched_long_decode", 64, 64, 8, 1, 32768, 128, 128,
                        seqlens=seqlens_loguniform(64, 1024, 32768),
                        note="batched long-context decode, KV lengths log-uniform [1024,32768], padded to 32768")
    raise ValueError(f"config index must be 1..5, got {idx}")

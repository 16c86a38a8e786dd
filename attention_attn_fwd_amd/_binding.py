"""ctypes binding of libattn_fwd.so (include/attn_fwd.h).

Argument marshalling only: every step of the attention forward runs in the
HIP kernels of the library.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_fwd.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_OOM, ATTN_ERR_HIP, ATTN_ERR_SCRATCH_LIMIT = range(6)
PATH_NONE, PATH_PREFILL, PATH_DECODE = 0, 1, 2
# attn_fwd_ex flags
ATTN_FWD_FP16, ATTN_FWD_FP32, ATTN_FWD_NONCAUSAL = 1, 2, 4

# Every function the header declares; a CPU test checks the library exports all of them.
EXPORTS = ("attn_fwd", "attn_fwd_f32", "attn_fwd_ex", "attn_fwd_noalloc", "attn_fwd_paged", "attn_bwd",
           "attn_fwd_strerror", "attn_fwd_plan", "attn_fwd_release_scratch")


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class _Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("split_workers", ctypes.c_int), ("partial_slots", ctypes.c_int),
                ("workspace_bytes", ctypes.c_int64)]


_lib = None


def load():
    """Load the HIP library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m attention_attn_fwd_amd.build` "
                              "(there is no fallback path)")
        # One HIP runtime per process: PyTorch ships its own libamdhip64 and
        # loads it by a name that does not match a runtime already mapped from
        # ROCm's lib directory, so loading the library first would leave two
        # runtimes side by side (the second one's launches can fail with
        # hipErrorNoDevice).  Loaded after torch, the library's dependency
        # resolves by soname to torch's copy.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        sig = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, cf, vp]
        lib.attn_fwd.argtypes = sig
        lib.attn_fwd.restype = ci
        lib.attn_fwd_f32.argtypes = sig
        lib.attn_fwd_f32.restype = ci
        lib.attn_fwd_ex.argtypes = sig[:-1] + [ci, vp]
        lib.attn_fwd_ex.restype = ci
        lib.attn_fwd_noalloc.argtypes = sig[:-1] + [ci, vp]
        lib.attn_fwd_noalloc.restype = ci
        lib.attn_fwd_paged.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, vp, ci, ci, ci, vp, ci, cf, ci, vp]
        lib.attn_fwd_paged.restype = ci
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, ci, cf, ci, vp]
        lib.attn_bwd.restype = ci
        lib.attn_fwd_strerror.argtypes = [ci]
        lib.attn_fwd_strerror.restype = ctypes.c_char_p
        lib.attn_fwd_plan.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(_Plan)]
        lib.attn_fwd_plan.restype = ci
        lib.attn_fwd_release_scratch.argtypes = []
        lib.attn_fwd_release_scratch.restype = ci
        _lib = lib
    return _lib


def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor, or an int / None passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None or isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream on ROCm


def strerror(status: int) -> str:
    return load().attn_fwd_strerror(int(status)).decode()


def attn_fwd_strerror(status: int) -> str:
    return strerror(status)


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, stream) -> int:
    """Raw C call (bf16).  Pointers may be tensors or ints; returns the status code."""
    return load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Q, K, D, Dv,
                           _ptr(seqlens_k), int(window), float(scale), _stream(stream))


def attn_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, stream) -> int:
    """Raw C call (fp32).  Pointers may be tensors or ints; returns the status code."""
    return load().attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Q, K, D, Dv,
                               _ptr(seqlens_k), int(window), float(scale), _stream(stream))


def attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, flags, stream) -> int:
    """Raw C call with option flags (ATTN_FWD_FP16 / _FP32 / _NONCAUSAL); returns the status."""
    return load().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Q, K, D, Dv,
                              _ptr(seqlens_k), int(window), float(scale), int(flags), _stream(stream))


def attn_fwd_noalloc(q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, flags, stream) -> int:
    """Raw C call of the entry point that allocates nothing (library-held scratch); returns the status."""
    return load().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Q, K, D, Dv,
                                   _ptr(seqlens_k), int(window), float(scale), int(flags), _stream(stream))


def attn_fwd_paged(q, k_pages, v_pages, o, lse, B, Hq, Hkv, Q, D, Dv, block_table, pages_per_seq, page_size,
                   num_pages, seqlens_k, window, scale, flags, stream) -> int:
    """Raw C call on a paged K/V cache; returns the status."""
    return load().attn_fwd_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), _ptr(lse), B, Hq, Hkv, Q, D, Dv,
                                 _ptr(block_table), int(pages_per_seq), int(page_size), int(num_pages),
                                 _ptr(seqlens_k), int(window), float(scale), int(flags), _stream(stream))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, flags,
             stream) -> int:
    """Raw C call of the backward; returns the status."""
    return load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                           B, Hq, Hkv, Q, K, D, Dv, _ptr(seqlens_k), int(window), float(scale), int(flags),
                           _stream(stream))


def attn_fwd_release_scratch() -> int:
    """Free the library's per-stream scratch buffers (waits for each device first); returns the status."""
    return load().attn_fwd_release_scratch()


def attn_fwd_plan(B, Hq, Hkv, Q, K, D, Dv, window=0) -> dict:
    plan = _Plan()
    st = load().attn_fwd_plan(B, Hq, Hkv, Q, K, D, Dv, int(window), ctypes.byref(plan))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_plan")
    return {"path": plan.path, "split_workers": plan.split_workers, "partial_slots": plan.partial_slots,
            "workspace_bytes": plan.workspace_bytes}


def forward(q, k, v, seqlens_k=None, window: int = 0, scale: Optional[float] = None, out=None, lse=None,
            stream=None, causal: bool = True):
    """GQA attention forward on torch tensors (causal unless causal=False).

    q [B,Hq,Q,D], k [B,Hkv,K,D], v [B,Hkv,K,Dv]: contiguous, on the GPU, all
    bfloat16 or all float16 (MFMA kernels, output in the input type) or all
    float32 (fp32 kernel).  seqlens_k: int32 [B] on the same device, or None.
    Returns (o, lse) with o [B,Hq,Q,Dv] in the input dtype and lse [B,Hq,Q]
    float32.
    """
    import torch

    if q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise TypeError("q, k, v must all be bfloat16, all float16 or all float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B,H,T,width]")
    B, Hq, Q, D = q.shape
    Bk, Hkv, K, Dk = k.shape
    Bv, Hv, Kv, Dv = v.shape
    if Bk != B or Bv != B or Hv != Hkv or Kv != K or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if seqlens_k is not None:
        if seqlens_k.dtype != torch.int32 or seqlens_k.device != q.device or tuple(seqlens_k.shape) != (B,):
            raise ValueError("seqlens_k must be int32 [B] on the same device")
        seqlens_k = seqlens_k.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Q, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Q), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    flags = {torch.bfloat16: 0, torch.float16: ATTN_FWD_FP16, torch.float32: ATTN_FWD_FP32}[q.dtype]
    if not causal:
        flags |= ATTN_FWD_NONCAUSAL
    st = attn_fwd_ex(q, k, v, out, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, flags, stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_ex")
    return out, lse


def forward_paged(q, k_pages, v_pages, block_table, seqlens_k=None, window: int = 0, scale: Optional[float] = None,
                  out=None, lse=None, stream=None, causal: bool = True):
    """Attention forward on a paged K/V cache (torch tensors on the GPU).

    q [B,Hq,Q,D]; k_pages [num_pages,Hkv,page_size,D], v_pages
    [num_pages,Hkv,page_size,Dv]; block_table int32 [B,pages_per_seq]: keys
    j*page_size.. of sequence b are in page block_table[b,j].  bfloat16 or
    float16.  Returns (o [B,Hq,Q,Dv], lse [B,Hq,Q] float32).
    """
    import torch

    if q.dtype != k_pages.dtype or q.dtype != v_pages.dtype or q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q, k_pages, v_pages must all be bfloat16 or all float16")
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, Hq, Q, D = q.shape
    num_pages, Hkv, page_size, Dk = k_pages.shape
    Dv = v_pages.shape[-1]
    if tuple(v_pages.shape[:3]) != (num_pages, Hkv, page_size) or Dk != D:
        raise ValueError(f"shape mismatch k_pages{tuple(k_pages.shape)} v_pages{tuple(v_pages.shape)}")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, pages_per_seq]")
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or tuple(seqlens_k.shape) != (B,)):
        raise ValueError("seqlens_k must be int32 [B] on the same device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Q, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Q), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    flags = (ATTN_FWD_FP16 if q.dtype == torch.float16 else 0) | (0 if causal else ATTN_FWD_NONCAUSAL)
    st = attn_fwd_paged(q, k_pages, v_pages, out, lse, B, Hq, Hkv, Q, D, Dv, block_table, block_table.shape[1],
                        page_size, num_pages, seqlens_k, window, scale, flags, stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_paged")
    return out, lse


def backward(q, k, v, o, lse, dout, seqlens_k=None, window: int = 0, scale: Optional[float] = None,
             stream=None, causal: bool = True):
    """Gradients of sum(dout * o) w.r.t. q, k, v on torch tensors (o and lse as the
    forward returned them).  bfloat16 or float16, D and Dv up to 256.
    Returns (dq, dk, dv) in the input dtype."""
    import torch

    if any(t.dtype != q.dtype for t in (k, v, o, dout)) or q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q, k, v, o, dout must all be bfloat16 or all float16")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, Hq, Q, D = q.shape
    _, Hkv, K, Dv = v.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    flags = (ATTN_FWD_FP16 if q.dtype == torch.float16 else 0) | (0 if causal else ATTN_FWD_NONCAUSAL)
    st = attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, flags,
                  torch.cuda.current_stream() if stream is None else stream)
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv

"""Helpers of the GPU parity tests: device buffers with guard bands, calls
through the C ABI, and comparison against the fp64 oracle."""
from __future__ import annotations

import hashlib
import sys

import numpy as np

import attention_attn_fwd_amd as af

DEV = "cuda:0"
# Maximum absolute error against the fp64 oracle, over every element.
# fp16 storage takes the bf16 bar: the same MFMA/fp32-accumulate path with a
# finer (10-bit) fraction on the inputs and weights.
TOL = {"bf16": {"o": 2e-2, "lse": 1e-3}, "f16": {"o": 2e-2, "lse": 1e-3}, "f32": {"o": 1e-4, "lse": 1e-4}}
GUARD = 4096  # bytes of canary after each output buffer


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)
    if arr.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t


def digest(t) -> str:
    import torch
    if t.numel() == 0:
        return hashlib.sha1(b"").hexdigest()
    return hashlib.sha1(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()


class Outputs:
    """O and LSE buffers prefilled with NaN, each followed by a 0xA5 canary band."""

    def __init__(self, w, dtype: str):
        import torch
        self.w, self.dtype = w, dtype
        esz = 4 if dtype == "f32" else 2
        n_o = int(np.prod(w.o_shape()))
        n_l = w.B * w.Hq * w.Q
        self.o_raw = torch.empty(n_o * esz + GUARD, dtype=torch.uint8, device=DEV)
        self.l_raw = torch.empty(n_l * 4 + GUARD, dtype=torch.uint8, device=DEV)
        self.o_raw[n_o * esz:].fill_(0xA5)
        self.l_raw[n_l * 4:].fill_(0xA5)
        if dtype in ("bf16", "f16"):
            self.o = self.o_raw[:n_o * esz].view(torch.bfloat16 if dtype == "bf16" else torch.float16)
            self.o.fill_(float("nan"))
        else:
            self.o = self.o_raw[:n_o * esz].view(torch.float32)
            self.o.fill_(float("nan"))
        self.l = self.l_raw[:n_l * 4].view(torch.float32)
        self.l.fill_(float("nan"))
        self.n_o, self.n_l, self.esz = n_o, n_l, esz

    def canaries_intact(self) -> bool:
        a = self.o_raw[self.n_o * self.esz:]
        b = self.l_raw[self.n_l * 4:]
        return bool((a == 0xA5).all().item()) and bool((b == 0xA5).all().item())

    def host(self):
        o = self.o.float().cpu().numpy().astype(np.float64).reshape(self.w.o_shape())
        lse = self.l.cpu().numpy().astype(np.float64).reshape(self.w.B, self.w.Hq, self.w.Q)
        return o, lse


def call(w, dq, dk, dv, dseq, outs: Outputs, scale=None, window=None, stream=None):
    """One call through the C ABI (attn_fwd / attn_fwd_f32, or attn_fwd_ex for fp16
    storage or the non-causal mode); returns the status."""
    import torch
    scale = w.scale if scale is None else scale
    window = w.window if window is None else window
    if stream is None:
        stream = torch.cuda.current_stream()
    causal = getattr(w, "causal", True)
    if w.dtype == "f16" or not causal:
        flags = {"bf16": 0, "f16": af.ATTN_FWD_FP16, "f32": af.ATTN_FWD_FP32}[w.dtype]
        if not causal:
            flags |= af.ATTN_FWD_NONCAUSAL
        return af.attn_fwd_ex(dq, dk, dv, outs.o, outs.l, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv, dseq, window,
                              scale, flags, stream)
    fn = af.attn_fwd if w.dtype == "bf16" else af.attn_fwd_f32
    return fn(dq, dk, dv, outs.o, outs.l, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv, dseq, window, scale, stream)


def run_gpu(w, q, k, v, *, scale=None, window=None, check_inputs=True, repeat_bitwise=True):
    """Run the GPU path on host arrays; returns (o, lse) as float64 host arrays.

    Checks: status OK, canaries intact, inputs bitwise unchanged, and (optionally)
    a second run into fresh NaN buffers is bitwise identical."""
    import torch
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    dseq = None if w.seqlens is None else to_dev(np.asarray(w.seqlens, np.int32))
    before = [digest(t) for t in (dq, dk, dv)] if check_inputs else None
    outs = Outputs(w, w.dtype)
    st = call(w, dq, dk, dv, dseq, outs, scale=scale, window=window)
    assert st == af.ATTN_OK, af.strerror(st)
    torch.cuda.synchronize()
    assert outs.canaries_intact(), "a kernel wrote past the end of O or LSE"
    if check_inputs:
        assert [digest(t) for t in (dq, dk, dv)] == before, "inputs were modified"
    o, lse = outs.host()
    if repeat_bitwise:
        outs2 = Outputs(w, w.dtype)
        st = call(w, dq, dk, dv, dseq, outs2, scale=scale, window=window)
        assert st == af.ATTN_OK
        torch.cuda.synchronize()
        assert torch.equal(outs.o_raw, outs2.o_raw), "second run differs bitwise (O)"
        assert torch.equal(outs.l_raw, outs2.l_raw), "second run differs bitwise (LSE)"
    return o, lse


def compare(o, lse, o_ref, lse_ref, dtype: str, what: str):
    """Max-abs comparison over every element; -inf must match exactly, no NaN anywhere."""
    tol = TOL[dtype]
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.isfinite(o).all(), f"{what}: Inf in O"
    ninf, ninf_ref = np.isneginf(lse), np.isneginf(lse_ref)
    assert np.array_equal(ninf, ninf_ref), f"{what}: -inf LSE pattern differs ({ninf.sum()} vs {ninf_ref.sum()})"
    assert not np.isposinf(lse).any()
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    fl = ~ninf
    err_l = float(np.max(np.abs(lse[fl] - lse_ref[fl]))) if fl.any() else 0.0
    say(f"  {what}: max|dO| = {err_o:.3e} (tol {tol['o']:.0e}), max|dLSE| = {err_l:.3e} (tol {tol['lse']:.0e})")
    assert err_o <= tol["o"], f"{what}: max abs O error {err_o:.3e} > {tol['o']}"
    assert err_l <= tol["lse"], f"{what}: max abs LSE error {err_l:.3e} > {tol['lse']}"
    return err_o, err_l

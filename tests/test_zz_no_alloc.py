"""attn_fwd_noalloc, the entry point for callers that cannot allocate device
memory, through the C ABI: bitwise the output of attn_fwd_ex on the same
inputs (same kernels and plan, the split-KV scratch held by the library), and
within the parity bar of the fp64 oracle, on two calls in a row, the second
smaller; a plan that needs more scratch than the library holds is refused
before anything runs; with every allocation forced to fail it still runs.
"""
import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as af
from attention_attn_fwd_amd import inputs
from gpu_util import Outputs, compare, say, to_dev

pytestmark = pytest.mark.gpu


def _call(fn, w, dev, outs, flags=0):
    q, k, v, seq = dev
    return fn(q, k, v, outs.o, outs.l, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv, seq, w.window, w.scale, flags,
              torch.cuda.current_stream())


def _both(w, orc, flags=0):
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    dev = (to_dev(q), to_dev(k), to_dev(v), None if w.seqlens is None else to_dev(w.seqlens))
    plan = af.attn_fwd_plan(*w.shape_tuple, window=w.window)
    say(f"[noalloc] {w.name} {w.shape_tuple} W={w.window} plan={plan}")
    assert plan["workspace_bytes"] > 0, "the case must use the split-KV scratch"
    ref, got = Outputs(w, w.dtype), Outputs(w, w.dtype)
    assert _call(af.attn_fwd_ex, w, dev, ref, flags) == af.ATTN_OK
    assert _call(af.attn_fwd_noalloc, w, dev, got, flags) == af.ATTN_OK
    torch.cuda.synchronize()
    assert got.canaries_intact()
    assert torch.equal(got.o_raw, ref.o_raw) and torch.equal(got.l_raw, ref.l_raw), "differs from attn_fwd_ex"
    o, lse = got.host()
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale, causal=w.causal)
    compare(o, lse, ro, rl, w.dtype, f"noalloc {w.name}")


def test_noalloc_two_calls_second_smaller(orc, monkeypatch):
    # Call 1: split-KV decode over long, unequal lengths (thousands of partial states).
    w1 = inputs.Workload("noalloc_decode", 8, 32, 8, 1, 8192, 128, 128,
                         seqlens=np.array([8192, 17, 4000, 0, 7777, 1, 6000, 2048], np.int32))
    _both(w1, orc)
    # Call 2, smaller: a prefill whose key ranges are cut into pieces (partial
    # states of 128-row tiles), fp16 storage, with a window.
    monkeypatch.setenv("ATTN_FWD_PREFILL_SPLITS", "3")
    w2 = inputs.Workload("noalloc_prefill", 1, 4, 2, 200, 1500, 64, 64, dtype="f16", window=300)
    _both(w2, orc, flags=af.ATTN_FWD_FP16)


def test_noalloc_refuses_plans_beyond_its_scratch(monkeypatch):
    # 100000 decode workers: 100000 x 8 rows x (128 + 2) floats of partial state, far past 64 MiB.
    monkeypatch.setenv("ATTN_FWD_SPLIT_WORKERS", "100000")
    w = inputs.Workload("noalloc_big", 1, 8, 1, 1, 4096, 128, 128)
    assert af.attn_fwd_plan(*w.shape_tuple)["workspace_bytes"] > 64 << 20
    dev = (to_dev(w.gen_q()), to_dev(w.gen_k()), to_dev(w.gen_v()), None)
    outs = Outputs(w, w.dtype)
    assert _call(af.attn_fwd_noalloc, w, dev, outs) == af.ATTN_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.isnan(outs.o.float()).all() and torch.isnan(outs.l).all(), "refused call wrote output"
    assert "64 MiB" in af.strerror(af.ATTN_ERR_SCRATCH_LIMIT)


def test_noalloc_needs_no_allocation(orc, monkeypatch):
    """With every scratch allocation forced to fail, attn_fwd_ex reports
    ATTN_ERR_OOM and attn_fwd_noalloc still runs and matches the oracle."""
    monkeypatch.setenv("ATTN_FWD_FAIL_ALLOC", "1")
    w = inputs.Workload("noalloc_failalloc", 2, 16, 4, 2, 3000, 80, 96, seqlens=np.array([3000, 1234], np.int32))
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    dev = (to_dev(q), to_dev(k), to_dev(v), to_dev(w.seqlens))
    outs = Outputs(w, w.dtype)
    assert _call(af.attn_fwd_ex, w, dev, outs) == af.ATTN_ERR_OOM
    assert _call(af.attn_fwd_noalloc, w, dev, outs) == af.ATTN_OK
    torch.cuda.synchronize()
    o, lse = outs.host()
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale)
    compare(o, lse, ro, rl, w.dtype, "noalloc under failing allocation")

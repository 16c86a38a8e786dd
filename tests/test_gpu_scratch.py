"""The scratch of the allocating entry points: one library-held buffer per
(device, stream), grown on demand.  Calls whose scratch fits return without
waiting for the GPU (they can be queued ahead of it); a call that needs more
grows the buffer; two streams never share one; results stay bitwise those of
attn_fwd_noalloc (same kernels and plan) and within the parity bar of the
fp64 oracle; attn_fwd_release_scratch frees the buffers and later calls
allocate again.
"""
import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as af
from attention_attn_fwd_amd import inputs
from gpu_util import Outputs, compare, say, to_dev

pytestmark = pytest.mark.gpu


def _dev(w):
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    return (q, k, v), (to_dev(q), to_dev(k), to_dev(v), None if w.seqlens is None else to_dev(w.seqlens))


def _call(fn, w, dev, outs, stream):
    q, k, v, seq = dev
    return fn(q, k, v, outs.o, outs.l, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv, seq, w.window, w.scale, 0, stream)


def _check(w, host, dev, outs, orc, what):
    """Bitwise attn_fwd_noalloc's result on the same inputs, and the oracle's bar."""
    ref = Outputs(w, w.dtype)
    assert _call(af.attn_fwd_noalloc, w, dev, ref, torch.cuda.current_stream()) == af.ATTN_OK
    torch.cuda.synchronize()
    assert outs.canaries_intact()
    assert torch.equal(outs.o_raw, ref.o_raw) and torch.equal(outs.l_raw, ref.l_raw), f"{what}: differs from noalloc"
    o, lse = outs.host()
    q, k, v = host
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale)
    compare(o, lse, ro, rl, w.dtype, what)


def test_split_calls_do_not_wait_for_the_gpu(orc):
    """With the stream's scratch already large enough, a split-KV decode call
    returns while earlier work on the stream is still running."""
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available in this build")
    w = inputs.Workload("scratch_async", 4, 16, 4, 1, 3000, 128, 128, seqlens=np.array([3000, 5, 1200, 0], np.int32))
    assert af.attn_fwd_plan(*w.shape_tuple)["workspace_bytes"] > 0
    host, dev = _dev(w)
    st = torch.cuda.current_stream()
    warm = Outputs(w, w.dtype)
    assert _call(af.attn_fwd_ex, w, dev, warm, st) == af.ATTN_OK  # sizes the stream's scratch
    torch.cuda.synchronize()
    outs = Outputs(w, w.dtype)
    torch.cuda._sleep(200_000_000)  # a bounded spin kernel ahead of the call on the same stream
    assert _call(af.attn_fwd_ex, w, dev, outs, st) == af.ATTN_OK
    pending = not st.query()
    torch.cuda.synchronize()
    say(f"[scratch] stream still busy when the call returned: {pending}")
    assert pending, "the call waited for the stream's earlier work"
    _check(w, host, dev, outs, orc, "queued split decode")


def test_scratch_grows_and_streams_do_not_share(orc):
    """Small, larger (the buffer grows), small again on one stream, with a
    second stream running other split calls concurrently; every output checked."""
    small = inputs.Workload("scratch_small", 2, 8, 2, 1, 700, 64, 64, seqlens=np.array([700, 33], np.int32))
    large = inputs.Workload("scratch_large", 16, 32, 8, 2, 9000, 128, 128,
                            seqlens=np.array([9000, 1, 8999, 4096, 0, 77, 5000, 6000,
                                              9000, 12, 3000, 4500, 2222, 8191, 64, 900], np.int32))
    other = inputs.Workload("scratch_other", 3, 12, 3, 3, 5000, 96, 80, seqlens=np.array([5000, 2500, 17], np.int32))
    plans = {w.name: af.attn_fwd_plan(*w.shape_tuple)["workspace_bytes"] for w in (small, large, other)}
    say(f"[scratch] workspace bytes {plans}")
    assert plans["scratch_large"] > 4 * plans["scratch_small"] > 0 and plans["scratch_other"] > 0
    data = {w.name: _dev(w) for w in (small, large, other)}
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    seq = (small, large, small)
    bufs = [(Outputs(w, w.dtype), Outputs(other, other.dtype)) for w in seq]
    torch.cuda.synchronize()  # the NaN fills ran on the default stream
    results = []
    for i, w in enumerate(seq):
        outs, outs2 = bufs[i]
        with torch.cuda.stream(s1):
            assert _call(af.attn_fwd_ex, w, data[w.name][1], outs, s1) == af.ATTN_OK
        with torch.cuda.stream(s2):
            assert _call(af.attn_fwd_ex, other, data[other.name][1], outs2, s2) == af.ATTN_OK
        results.append((w, outs, f"{w.name} call {i} on stream 1"))
        results.append((other, outs2, f"{other.name} call {i} on stream 2"))
    torch.cuda.synchronize()
    for w, outs, what in results:
        _check(w, data[w.name][0], data[w.name][1], outs, orc, what)


def test_release_then_call_again(orc):
    w = inputs.Workload("scratch_release", 2, 8, 2, 1, 2500, 128, 128, seqlens=np.array([2500, 1300], np.int32))
    host, dev = _dev(w)
    st = torch.cuda.current_stream()
    a = Outputs(w, w.dtype)
    assert _call(af.attn_fwd_ex, w, dev, a, st) == af.ATTN_OK
    assert af.attn_fwd_release_scratch() == af.ATTN_OK  # waits for the call above
    assert af.attn_fwd_release_scratch() == af.ATTN_OK  # nothing held: a no-op
    _check(w, host, dev, a, orc, "before the release")
    b = Outputs(w, w.dtype)
    assert _call(af.attn_fwd_ex, w, dev, b, st) == af.ATTN_OK
    torch.cuda.synchronize()
    _check(w, host, dev, b, orc, "after the release")


def test_captured_call_replays_match_eager(orc):
    """A split-KV decode call captured into a HIP graph (after one call of the
    same size has sized the capturing stream's scratch) replays three times,
    with eager calls on the same stream between replays; every replay is
    bitwise the eager result."""
    w = inputs.Workload("scratch_graph", 4, 16, 4, 1, 2600, 128, 128, seqlens=np.array([2600, 9, 1500, 0], np.int32))
    assert af.attn_fwd_plan(*w.shape_tuple)["workspace_bytes"] > 0
    host, dev = _dev(w)
    s = torch.cuda.Stream()
    eager, graphed = Outputs(w, w.dtype), Outputs(w, w.dtype)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        assert _call(af.attn_fwd_ex, w, dev, eager, s) == af.ATTN_OK  # sizes s's scratch
    torch.cuda.synchronize()
    _check(w, host, dev, eager, orc, "eager before capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = _call(af.attn_fwd_ex, w, dev, graphed, s)
    assert st == af.ATTN_OK
    for i in range(3):
        graphed.o.fill_(float("nan"))
        graphed.l.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
            other = Outputs(w, w.dtype)
            torch.cuda.synchronize()
            assert _call(af.attn_fwd_ex, w, dev, other, s) == af.ATTN_OK  # an eager call between replays
        torch.cuda.synchronize()
        say(f"[scratch] replay {i}")
        assert torch.equal(graphed.o_raw, eager.o_raw) and torch.equal(graphed.l_raw, eager.l_raw), f"replay {i}"
        assert torch.equal(other.o_raw, eager.o_raw) and torch.equal(other.l_raw, eager.l_raw), f"eager {i}"

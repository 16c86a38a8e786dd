"""Backward (attn_bwd) against the fp64 oracle's gradients.

Each case runs the GPU forward (attn_fwd_ex) for O and LSE, then attn_bwd with
a seeded dO, into NaN-prefilled dQ/dK/dV buffers followed by canary bands, and
compares with the oracle's gradients of sum(dO * O) computed in fp64 from the
same rounded inputs.  The bar, per tensor: max |gpu - oracle| <= 2e-2 *
max(1, max |oracle|) (bf16 and fp16 storage; the weights and dS are rounded to
the storage type for the products and the outputs are rounded once, each a
relative 2^-9, summed over rows or keys with varying signs).  Every element
must be written (no NaN left), canaries intact, inputs unchanged, and a second
call bitwise identical.
"""
import numpy as np
import pytest

import attention_attn_fwd_amd as af
from attention_attn_fwd_amd import inputs
from gpu_util import GUARD, DEV, Outputs, call, digest, say, to_dev

pytestmark = pytest.mark.gpu

DOUT_ID = 7  # input stream of dO
TOL = 2e-2


def _guarded(shape, dtype):
    import torch
    n = int(np.prod(shape))
    raw = torch.empty(n * 2 + GUARD, dtype=torch.uint8, device=DEV)
    raw[n * 2:].fill_(0xA5)
    t = raw[:n * 2].view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    t.fill_(float("nan"))
    return raw, t


def _flags(w):
    return (af.ATTN_FWD_FP16 if w.dtype == "f16" else 0) | (0 if w.causal else af.ATTN_FWD_NONCAUSAL)


def _check(orc, w, scale=None, window=None, tag=""):
    import torch
    scale = w.scale if scale is None else scale
    window = w.window if window is None else window
    say(f"[bwd] {w.name} {w.shape_tuple} {w.dtype} causal={w.causal} W={window} scale={scale} "
        f"seqlens={None if w.seqlens is None else list(w.seqlens)} {tag}")
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    dout = inputs.normal(w.o_shape(), DOUT_ID, w.seed, w.dtype)
    dq_in, dk_in, dv_in, do_in = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    dseq = None if w.seqlens is None else to_dev(np.asarray(w.seqlens, np.int32))
    outs = Outputs(w, w.dtype)
    assert call(w, dq_in, dk_in, dv_in, dseq, outs, scale=scale, window=window) == af.ATTN_OK
    before = [digest(t) for t in (dq_in, dk_in, dv_in, do_in, outs.o, outs.l)]
    results = []
    for _ in range(2):
        gq_raw, gq = _guarded(w.q_shape(), w.dtype)
        gk_raw, gk = _guarded(w.k_shape(), w.dtype)
        gv_raw, gv = _guarded(w.v_shape(), w.dtype)
        st = af.attn_bwd(dq_in, dk_in, dv_in, outs.o, outs.l, do_in, gq, gk, gv, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D,
                         w.Dv, dseq, window, scale, _flags(w), torch.cuda.current_stream())
        assert st == af.ATTN_OK, af.strerror(st)
        torch.cuda.synchronize()
        for raw, t in ((gq_raw, gq), (gk_raw, gk), (gv_raw, gv)):
            assert bool((raw[t.numel() * 2:] == 0xA5).all().item()), "a kernel wrote past the end of a gradient"
        results.append((gq, gk, gv))
    assert [digest(t) for t in (dq_in, dk_in, dv_in, do_in, outs.o, outs.l)] == before, "inputs were modified"
    for a, b in zip(results[0], results[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "second call differs bitwise"
    rq, rk, rv = orc.bwd(q, k, v, dout, seqlens=w.seqlens, window=window, scale=scale, causal=w.causal)
    errs = {}
    for name, g, r in (("dq", results[0][0], rq), ("dk", results[0][1], rk), ("dv", results[0][2], rv)):
        gh = g.float().cpu().numpy().astype(np.float64).reshape(r.shape)
        assert not np.isnan(gh).any(), f"{name}: an element was not written (NaN left)"
        ref_max = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(gh - r))) if r.size else 0.0
        errs[name] = (err, ref_max)
        assert err <= TOL * max(1.0, ref_max), f"{name}: max abs err {err:.3e} vs max|ref| {ref_max:.3e}"
    say("       " + "  ".join(f"{n}: err {e:.2e} (max|ref| {m:.2e})" for n, (e, m) in errs.items()))
    return errs


SHAPES = [
    (1, 4, 2, 64, 128, 64, 64),
    (1, 4, 2, 65, 131, 64, 64),
    (2, 8, 2, 300, 300, 128, 128),
    (1, 8, 2, 256, 1024, 64, 64),
    (1, 4, 1, 200, 700, 128, 64),
    (1, 4, 2, 130, 90, 64, 128),     # more rows than keys
    (1, 8, 2, 1, 2053, 80, 96),      # one query row, padded widths
    (3, 6, 3, 2, 777, 16, 32),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes(orc, shape, dtype, causal):
    _check(orc, inputs.Workload("bwd", *shape, dtype=dtype, causal=causal))


# Heads wider than 128 (up to 256, padded to 256): dK and dV in separate
# launches, one dQ workgroup per CU.
WIDE = [
    (1, 4, 2, 64, 128, 256, 256),
    (2, 8, 2, 200, 300, 256, 256),
    (1, 8, 2, 1, 999, 192, 256),
    (1, 4, 4, 130, 90, 256, 128),
    (2, 4, 2, 65, 131, 144, 80),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "x".join(map(str, s)))
def test_bwd_wide_heads(orc, shape, dtype, causal):
    _check(orc, inputs.Workload("bwd_wide", *shape, dtype=dtype, causal=causal))
    if causal and shape[0] > 1:
        sl = np.array([shape[4], 0][:shape[0]], np.int32)
        _check(orc, inputs.Workload("bwd_wide_varlen", *shape, dtype=dtype, seqlens=sl), window=33, tag=" W=33")


@pytest.mark.parametrize("window", [1, 17, 64, 200])
def test_bwd_window(orc, window):
    sl = np.array([333, 0, 100], np.int32)
    _check(orc, inputs.Workload("bwd_window", 3, 4, 2, 200, 333, 64, 64, window=window, seqlens=sl))


@pytest.mark.parametrize("Q", [1, 3, 160])
def test_bwd_varlen(orc, Q):
    sl = np.array([0, 1, 7, 64, 129, 160, 33, 0], np.int32)
    _check(orc, inputs.Workload("bwd_varlen", 8, 8, 2, Q, 160, 64, 64, seqlens=sl))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_bwd_scales(orc, scale):
    _check(orc, inputs.Workload("bwd_scale", 1, 4, 2, 77, 190, 64, 64), scale=scale)


def test_bwd_empty_keys(orc):
    """Every K_b = 0: no row has a key, every gradient is 0."""
    _check(orc, inputs.Workload("bwd_nokeys", 2, 4, 2, 5, 64, 64, 64, seqlens=np.array([0, 0], np.int32)))


def test_bwd_backward_api(orc):
    """The torch-level backward() wrapper on the same call."""
    import torch
    w = inputs.Workload("bwd_api", 2, 8, 2, 100, 300, 64, 64, dtype="f16", seqlens=np.array([300, 50], np.int32))
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    dout = inputs.normal(w.o_shape(), DOUT_ID, w.seed, w.dtype)
    tq, tk, tv, td = (to_dev(a) for a in (q, k, v, dout))
    sl = to_dev(w.seqlens)
    o, lse = af.forward(tq, tk, tv, seqlens_k=sl)
    dq, dk, dv = af.backward(tq, tk, tv, o, lse, td, seqlens_k=sl)
    torch.cuda.synchronize()
    rq, rk, rv = orc.bwd(q, k, v, dout, seqlens=w.seqlens)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = float(np.max(np.abs(g.float().cpu().numpy() - r)))
        assert err <= TOL * max(1.0, float(np.max(np.abs(r)))), (name, err)


def test_bwd_full_dense_prefill_shape(orc):
    """The backward at the dense prefill shape the bench times (B=4, Hq=32,
    Hkv=8, Q=K=4096, D=Dv=128), on samples: dq of 256 rows (tile edges and
    random ones) and dk/dv of 48 keys in three (batch, kv-head) groups, from
    the oracle's sampled backward; every element written and finite."""
    import torch
    w = inputs.config(3)
    say(f"[bwd] full {w.name} {w.shape_tuple}")
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    dout = inputs.normal(w.o_shape(), DOUT_ID, w.seed, "bf16")
    tq, tk, tv, td = (to_dev(a) for a in (q, k, v, dout))
    o, lse = af.forward(tq, tk, tv)
    dq, dk, dv = af.backward(tq, tk, tv, o, lse, td)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all().item()), f"{name}: non-finite or unwritten elements"
    rng = np.random.default_rng(3)
    rows = set()
    for qq in (0, 127, 128, 2047, 4095):
        for b in range(w.B):
            rows.add((b * w.Hq + int(rng.integers(w.Hq))) * w.Q + qq)
    while len(rows) < 256:
        rows.add(int(rng.integers(w.B * w.Hq * w.Q)))
    rows = np.array(sorted(rows), np.int64)
    keys = []
    for gi in (0, 13, 31):
        for kk in (0, 63, 64, 127, 128, 4032, 4095):
            keys.append(gi * w.K + kk)
        keys += [gi * w.K + int(x) for x in rng.integers(0, w.K, 9)]
    keys = np.array(sorted(set(keys)), np.int64)
    rq = orc.bwd_rows(q, k, v, dout, rows)
    rk, rv = orc.bwd_keys(q, k, v, dout, keys)
    gq = dq.float().cpu().numpy().reshape(-1, w.D)[rows]
    gk = dk.float().cpu().numpy().reshape(-1, w.D)[keys]
    gv = dv.float().cpu().numpy().reshape(-1, w.Dv)[keys]
    for name, g, r in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        err = float(np.max(np.abs(g - r)))
        ref_max = float(np.max(np.abs(r)))
        say(f"       {name}: err {err:.2e} (max|ref| {ref_max:.2e}, {len(r)} sampled)")
        assert err <= TOL * max(1.0, ref_max), f"{name}: max abs err {err:.3e} vs max|ref| {ref_max:.3e}"


def test_bwd_forced_scratch_failure_reports_oom():
    """A failed scratch allocation is reported; nothing is written."""
    import os
    import torch
    w = inputs.Workload("bwd_oom", 1, 4, 2, 40, 100, 64, 64)
    q, k, v = (to_dev(a) for a in (w.gen_q(), w.gen_k(), w.gen_v()))
    o, lse = af.forward(q, k, v)
    dout = to_dev(inputs.normal(w.o_shape(), DOUT_ID, w.seed, "bf16"))
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    os.environ["ATTN_FWD_FAIL_ALLOC"] = "1"
    try:
        st = af.attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv, None, 0, w.scale,
                         0, torch.cuda.current_stream())
    finally:
        del os.environ["ATTN_FWD_FAIL_ALLOC"]
    torch.cuda.synchronize()
    assert st == af.ATTN_ERR_OOM
    for t in (dq, dk, dv):
        assert torch.isnan(t.float()).all()


def test_bwd_side_stream(orc):
    """The backward on a side stream, waited on by the default stream."""
    import torch
    w = inputs.Workload("bwd_stream", 2, 8, 2, 130, 700, 128, 128, seqlens=np.array([700, 301], np.int32))
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    dout = inputs.normal(w.o_shape(), DOUT_ID, w.seed, "bf16")
    tq, tk, tv, td, sl = (to_dev(a) for a in (q, k, v, dout, w.seqlens))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o, lse = af.forward(tq, tk, tv, seqlens_k=sl, stream=side)
        dq, dk, dv = af.backward(tq, tk, tv, o, lse, td, seqlens_k=sl, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    refs = orc.bwd(q, k, v, dout, seqlens=w.seqlens)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = float(np.max(np.abs(g.float().cpu().numpy() - r)))
        assert err <= TOL * max(1.0, float(np.max(np.abs(r)))), (name, err)

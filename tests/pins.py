"""Pins of the fp64 oracle against facts fixed outside it.

Each pin takes an oracle object (oracle.attn_oracle.Oracle) and raises
AssertionError when the oracle disagrees with:
  - hand-derived worked examples (tests/golden/worked_examples.json),
  - textbook causal attention as computed by torch's scaled_dot_product_attention
    in float64 on the CPU (a library routine),
  - closed forms (uniform V, a single legal key, zero scale),
  - numpy's float16 conversion (every finite binary16 pattern),
  - torch's unmasked attention for the non-causal mode, and key-order
    independence there,
  - invariants (shift of K along a fixed direction, weights summing to one,
    split-and-merge by log-sum-exp, GQA equal to MHA on repeated heads,
    padding never read, V/O columns beyond Dv never touched).
The definition pinned is the attention fixture of the LuisaCompute "Attention
execution mapping" review, section 1 (bottom-right causal GQA, kv-head
h/(Hq/Hkv), legal keys k <= q + K - Q, online state carried across KV blocks),
with the per-sequence-length and window readings stated in the design notes.

The mutation test runs INDEPENDENT_PINS on oracle builds with one planted
mistake each and requires every build to fail at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    ninf_a, ninf_b = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ninf_a, ninf_b), f"{what}: -inf pattern differs"
    fa, fb = a[~ninf_a], b[~ninf_b]
    assert np.all(np.isfinite(fa)), f"{what}: non-finite values"
    err = float(np.max(np.abs(fa - fb))) if fa.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _sdpa_causal_square(q, k, v, scale):
    """Textbook lower-triangular causal attention (Q == K) via torch, float64, CPU.
    Returns (o, lse) with kv heads repeated over their query groups."""
    tq = torch.from_numpy(q.astype(np.float64))
    tk = torch.from_numpy(k.astype(np.float64))
    tv = torch.from_numpy(v.astype(np.float64))
    g = tq.shape[1] // tk.shape[1]
    tk = tk.repeat_interleave(g, dim=1)
    tv = tv.repeat_interleave(g, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    n = tq.shape[2]
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    tri = torch.ones(n, n, dtype=torch.bool).tril()
    s = s.masked_fill(~tri, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


# ---------------------------------------------------------------- worked examples
def pin_worked_examples(orc):
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=np.float32)
    k = np.array(ex["k"], dtype=np.float32)
    v = np.array(ex["v"], dtype=np.float32)
    assert ex["scale"] == "ln3"
    for case in ex["cases"]:
        sl = None if case["seqlens"] is None else np.array(case["seqlens"], dtype=np.int32)
        o, lse = orc.fwd(q, k, v, seqlens=sl, window=case["window"], scale=math.log(3.0))
        want_o = np.array([[[[float(Fraction(x)) for x in row] for row in head] for head in bat]
                           for bat in case["o"]])
        want_lse = np.array([[[(-math.inf if x == "-inf" else math.log(Fraction(x[3:]))) for x in head]
                              for head in bat] for bat in case["lse"]])
        _close(o, want_o, 1e-12, f"worked example {case['name']} O")
        _close(lse, want_lse, 1e-12, f"worked example {case['name']} LSE")


# ---------------------------------------------------------------- textbook / library
def pin_textbook_causal(orc):
    rng = np.random.default_rng(11)
    for (B, Hq, Hkv, N, D, Dv) in [(2, 4, 2, 37, 16, 24), (1, 3, 3, 20, 8, 8), (1, 4, 1, 33, 32, 16)]:
        q, k, v = _f32(rng, (B, Hq, N, D)), _f32(rng, (B, Hkv, N, D)), _f32(rng, (B, Hkv, N, Dv))
        scale = 1.0 / math.sqrt(D)
        o, lse = orc.fwd(q, k, v, scale=scale)
        ro, rl = _sdpa_causal_square(q, k, v, scale)
        _close(o, ro, 1e-12, f"textbook causal O {B,Hq,Hkv,N,D,Dv}")
        _close(lse, rl, 1e-12, f"textbook causal LSE {B,Hq,Hkv,N,D,Dv}")


def pin_bottom_right(orc):
    """Q < K rows are the last Q rows of the square causal problem (decode included)."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, K, D, Dv = 1, 4, 2, 29, 16, 8
    qf, k, v = _f32(rng, (B, Hq, K, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    scale = 0.37
    ro, rl = _sdpa_causal_square(qf, k, v, scale)
    for Q in (1, 2, 5, 17):
        q = np.ascontiguousarray(qf[:, :, K - Q:, :])
        o, lse = orc.fwd(q, k, v, scale=scale)
        _close(o, ro[:, :, K - Q:, :], 1e-12, f"bottom-right Q={Q} O")
        _close(lse, rl[:, :, K - Q:], 1e-12, f"bottom-right Q={Q} LSE")


# ---------------------------------------------------------------- closed forms
def pin_uniform_v(orc):
    rng = np.random.default_rng(13)
    B, Hq, Hkv, Q, K, D, Dv = 2, 4, 2, 7, 19, 16, 12
    q, k = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D))
    row = _f32(rng, (B, Hkv, 1, Dv))
    v = np.ascontiguousarray(np.broadcast_to(row, (B, Hkv, K, Dv)))
    for window, sl in [(0, None), (3, None), (0, np.array([19, 4], np.int32))]:
        o, lse = orc.fwd(q, k, v, seqlens=sl, window=window)
        want = np.repeat(np.repeat(row.astype(np.float64), Hq // Hkv, axis=1), Q, axis=2)
        has = np.isfinite(lse)
        assert has.any()
        _close(o[has], want[has], 1e-12, "uniform V gives V")


def pin_single_key(orc):
    """Window 1, or K_b = 1 at the last row: O is that key's V row and LSE its score."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, Q, K, D, Dv = 1, 4, 2, 6, 11, 16, 8
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    scale = 0.5
    o, lse = orc.fwd(q, k, v, window=1, scale=scale)
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        for i in range(Q):
            p = i + K - Q
            _close(o[0, h, i], v[0, kh, p], 1e-12, "window 1 O")
            want = scale * float(np.dot(q[0, h, i].astype(np.float64), k[0, kh, p].astype(np.float64)))
            _close(lse[0, h, i], want, 1e-12, "window 1 LSE")
    o, lse = orc.fwd(q, k, v, seqlens=np.array([1], np.int32), scale=scale)
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        _close(o[0, h, Q - 1], v[0, kh, 0], 1e-12, "K_b = 1 O")
        want = scale * float(np.dot(q[0, h, Q - 1].astype(np.float64), k[0, kh, 0].astype(np.float64)))
        _close(lse[0, h, Q - 1], want, 1e-12, "K_b = 1 LSE")


def pin_scale_zero(orc):
    """scale 0: uniform weights over the legal keys, so O is their mean and LSE ln(count)."""
    rng = np.random.default_rng(15)
    B, Hq, Hkv, N, D, Dv = 1, 2, 1, 23, 8, 8
    q, k, v = _f32(rng, (B, Hq, N, D)), _f32(rng, (B, Hkv, N, D)), _f32(rng, (B, Hkv, N, Dv))
    vd = v.astype(np.float64)
    for window in (0, 5):
        o, lse = orc.fwd(q, k, v, window=window, scale=0.0)
        for i in range(N):
            lo = 0 if window <= 0 else max(0, i - window + 1)
            want = vd[0, 0, lo:i + 1].mean(axis=0)
            for h in range(Hq):
                _close(o[0, h, i], want, 1e-12, f"scale 0 O (window {window})")
                _close(lse[0, h, i], math.log(i + 1 - lo), 1e-12, f"scale 0 LSE (window {window})")


def pin_empty_rows(orc):
    rng = np.random.default_rng(16)
    B, Hq, Hkv, Q, K, D, Dv = 3, 2, 1, 9, 6, 8, 8
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    sl = np.array([0, 6, 2], np.int32)
    o, lse = orc.fwd(q, k, v, seqlens=sl)
    for b in range(B):
        for i in range(Q):
            empty = (i + sl[b] - Q) < 0   # no key at or before the row's position
            if empty:
                assert np.all(o[b, :, i] == 0.0), "empty row O must be 0"
                assert np.all(np.isneginf(lse[b, :, i])), "empty row LSE must be -inf"
            else:
                assert np.all(np.isfinite(lse[b, :, i])), "row with keys must have finite LSE"
    assert np.all(np.isfinite(o))


# ---------------------------------------------------------------- invariants
def pin_shift_invariance(orc):
    """K' = K + 1 u^T: weights unchanged, LSE moves by scale * q.u (exact inputs on a 1/8 grid)."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, Q, K, D, Dv = 1, 4, 2, 5, 13, 16, 8
    grid = lambda shape: (rng.integers(-8, 9, size=shape) / 8.0).astype(np.float32)
    q, k, v = grid((B, Hq, Q, D)), grid((B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    u = grid((B, Hkv, 1, D))
    u[..., -1] = 0.75
    k2 = np.ascontiguousarray(k + u)
    scale = 0.25
    o1, l1 = orc.fwd(q, k, v, scale=scale, window=4)
    o2, l2 = orc.fwd(q, k2, v, scale=scale, window=4)
    _close(o2, o1, 1e-12, "shift invariance O")
    g = Hq // Hkv
    ur = np.repeat(u.astype(np.float64), g, axis=1)[:, :, 0, :]
    shift = scale * np.einsum("bhqd,bhd->bhq", q.astype(np.float64), ur)
    _close(l2, l1 + shift, 1e-12, "shift invariance LSE")


def pin_probs_sum_to_one(orc):
    rng = np.random.default_rng(18)
    B, Hq, Hkv, Q, K, D = 2, 4, 2, 8, 21, 16
    q, k = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D))
    sl = np.array([21, 5], np.int32)
    for b in range(B):
        for h in range(Hq):
            for i in range(Q):
                p, n = orc.probs(q, k, b, h, i, seqlens=sl, window=6)
                assert np.all(p >= 0.0)
                assert np.count_nonzero(p) <= n
                if n:
                    assert abs(math.fsum(p) - 1.0) <= 1e-13, "weights must sum to 1"
                else:
                    assert not p.any()


def pin_split_merge(orc):
    """Attention over [0,K) equals the log-sum-exp merge of [0,s) and [s,K)."""
    rng = np.random.default_rng(19)
    Hq, Hkv, K, D, Dv = 2, 1, 40, 16, 8
    q, k, v = _f32(rng, (1, Hq, 1, D)), _f32(rng, (1, Hkv, K, D)), _f32(rng, (1, Hkv, K, Dv))
    of, lf = orc.fwd(q, k, v)
    for s in (1, 17, 39):
        o1, l1 = orc.fwd(q, np.ascontiguousarray(k[:, :, :s]), np.ascontiguousarray(v[:, :, :s]))
        o2, l2 = orc.fwd(q, np.ascontiguousarray(k[:, :, s:]), np.ascontiguousarray(v[:, :, s:]))
        m = np.maximum(l1, l2)
        w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
        om = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
        lm = m + np.log(w1 + w2)
        _close(om, of, 1e-12, f"split-merge O at {s}")
        _close(lm, lf, 1e-12, f"split-merge LSE at {s}")


def pin_gqa_expand(orc):
    rng = np.random.default_rng(20)
    B, Hq, Hkv, Q, K, D, Dv = 2, 8, 2, 6, 15, 16, 8
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    sl = np.array([15, 9], np.int32)
    o, lse = orc.fwd(q, k, v, seqlens=sl, window=7)
    g = Hq // Hkv
    ke, ve = np.ascontiguousarray(np.repeat(k, g, axis=1)), np.ascontiguousarray(np.repeat(v, g, axis=1))
    o2, l2 = orc.fwd(q, ke, ve, seqlens=sl, window=7)
    _close(o, o2, 0.0, "GQA equals MHA on repeated kv heads (O)")
    _close(lse, l2, 0.0, "GQA equals MHA on repeated kv heads (LSE)")


def pin_varlen_unpadded(orc):
    """A padded batch entry equals its own unpadded run; NaN padding is never read."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, Q, K, D, Dv = 3, 4, 2, 5, 14, 16, 8
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    sl = np.array([14, 3, 8], np.int32)
    kp, vp = k.copy(), v.copy()
    for b in range(B):
        kp[b, :, sl[b]:] = np.nan
        vp[b, :, sl[b]:] = np.nan
    o, lse = orc.fwd(q, kp, vp, seqlens=sl)
    o_clean, lse_clean = orc.fwd(q, k, v, seqlens=sl)
    _close(o, o_clean, 0.0, "NaN padding changes nothing (O)")
    _close(lse, lse_clean, 0.0, "NaN padding changes nothing (LSE)")
    for b in range(B):
        Kb = int(sl[b])
        ob, lb = orc.fwd(np.ascontiguousarray(q[b:b + 1]), np.ascontiguousarray(k[b:b + 1, :, :Kb]),
                         np.ascontiguousarray(v[b:b + 1, :, :Kb]))
        _close(o[b:b + 1], ob, 0.0, f"varlen entry {b} equals its unpadded run (O)")
        _close(lse[b:b + 1], lb, 0.0, f"varlen entry {b} equals its unpadded run (LSE)")


def pin_v_columns_untouched(orc):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, Q, K, D, Dv = 1, 2, 1, 4, 9, 8, 6
    q, k = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D))
    vw = np.full((B, Hkv, K, Dv + 5), np.nan, dtype=np.float32)
    vw[..., :Dv] = _f32(rng, (B, Hkv, K, Dv))
    ow = np.full((B, Hq, Q, Dv + 3), 7.25)
    lse = np.empty((B, Hq, Q))
    orc.fwd_into(q, k, vw, ow, lse, D=D, Dv=Dv)
    assert np.all(ow[..., Dv:] == 7.25), "O columns beyond Dv were written"
    assert np.all(np.isfinite(ow[..., :Dv])), "V columns beyond Dv leaked into O"
    o_ref, l_ref = orc.fwd(q, k, np.ascontiguousarray(vw[..., :Dv]))
    _close(ow[..., :Dv], o_ref, 0.0, "wide-row O equals narrow-row O")


# ---------------------------------------------------------------- fp16 storage
def pin_fp16_decode(orc):
    """Every finite IEEE binary16 pattern is read as its exact value: batch b is a
    one-row, one-key problem with q = pattern b, k = 1.0 and scale 1, so its LSE is
    q itself; numpy's float16 -> float64 conversion is the reference."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    bits = bits[np.isfinite(vals)]
    n = len(bits)
    q = bits.view(np.float16).reshape(n, 1, 1, 1).copy()
    k = np.ones((n, 1, 1, 1), dtype=np.float16)
    v = np.ones((n, 1, 1, 1), dtype=np.float16)
    o, lse = orc.fwd(q, k, v, scale=1.0)
    want = q.astype(np.float64).reshape(n, 1, 1)
    assert np.array_equal(lse, want), "fp16 inputs must decode exactly"
    assert np.all(o == 1.0)


# ---------------------------------------------------------------- non-causal
def _sdpa_full(q, k, v, scale, kb=None):
    """Attention without a mask via torch (float64, CPU), kv heads repeated over their
    query groups; kb limits every batch entry to its first kb[b] keys."""
    B = q.shape[0]
    g = q.shape[1] // k.shape[1]
    outs, lses = [], []
    for b in range(B):
        n = k.shape[2] if kb is None else int(kb[b])
        tq = torch.from_numpy(q[b:b + 1].astype(np.float64))
        if n == 0:
            outs.append(np.zeros(q[b:b + 1].shape[:3] + (v.shape[-1],)))
            lses.append(np.full(q[b:b + 1].shape[:3], -np.inf))
            continue
        tk = torch.from_numpy(k[b:b + 1, :, :n].astype(np.float64)).repeat_interleave(g, dim=1)
        tv = torch.from_numpy(v[b:b + 1, :, :n].astype(np.float64)).repeat_interleave(g, dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False, scale=scale)
        s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        outs.append(o.numpy())
        lses.append(torch.logsumexp(s, dim=-1).numpy())
    return np.concatenate(outs), np.concatenate(lses)


def pin_noncausal_textbook(orc):
    """causal=False is plain (unmasked) attention over each entry's first K_b keys."""
    rng = np.random.default_rng(24)
    for (B, Hq, Hkv, Q, K, D, Dv, sl) in [(2, 4, 2, 7, 19, 16, 8, None), (1, 3, 1, 21, 5, 8, 12, None),
                                          (3, 4, 2, 1, 13, 16, 16, [13, 0, 4]), (2, 2, 2, 9, 9, 7, 5, [3, 9])]:
        q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
        scale = 0.3
        sla = None if sl is None else np.array(sl, np.int32)
        o, lse = orc.fwd(q, k, v, seqlens=sla, scale=scale, causal=False)
        ro, rl = _sdpa_full(q, k, v, scale, sla)
        _close(o, ro, 1e-12, f"non-causal O {B,Hq,Hkv,Q,K,D,Dv,sl}")
        _close(lse, rl, 1e-12, f"non-causal LSE {B,Hq,Hkv,Q,K,D,Dv,sl}")


def pin_noncausal_key_order(orc):
    """Without the causal limit the keys form a set: permuting the first K_b rows of K
    and V together changes nothing (with the limit it would)."""
    rng = np.random.default_rng(25)
    B, Hq, Hkv, Q, K, D, Dv = 2, 4, 2, 6, 17, 16, 8
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    sl = np.array([17, 11], np.int32)
    o1, l1 = orc.fwd(q, k, v, seqlens=sl, causal=False)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        perm = rng.permutation(int(sl[b]))
        k2[b, :, :sl[b]] = k[b][:, perm]
        v2[b, :, :sl[b]] = v[b][:, perm]
    o2, l2 = orc.fwd(q, k2, v2, seqlens=sl, causal=False)
    _close(o2, o1, 1e-12, "non-causal key permutation O")
    _close(l2, l1, 1e-12, "non-causal key permutation LSE")


def pin_noncausal_closed_forms(orc):
    """causal=False, scale 0: O is the mean of the first K_b V rows, LSE ln K_b (every
    row, whatever its position); K_b = 0 rows give O = 0, LSE = -inf."""
    rng = np.random.default_rng(26)
    B, Hq, Hkv, Q, K, D, Dv = 3, 2, 1, 5, 9, 8, 6
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    sl = np.array([9, 2, 0], np.int32)
    o, lse = orc.fwd(q, k, v, seqlens=sl, scale=0.0, causal=False)
    vd = v.astype(np.float64)
    for b in range(B):
        n = int(sl[b])
        for h in range(Hq):
            for i in range(Q):
                if n == 0:
                    assert np.all(o[b, h, i] == 0.0) and np.isneginf(lse[b, h, i]), "K_b = 0 row"
                else:
                    _close(o[b, h, i], vd[b, 0, :n].mean(axis=0), 1e-12, "non-causal scale 0 O")
                    _close(lse[b, h, i], math.log(n), 1e-12, "non-causal scale 0 LSE")


def pin_noncausal_needs_no_window(orc):
    """A window is measured back from the diagonal, so it needs the causal limit."""
    q = np.zeros((1, 1, 1, 8), np.float32)
    try:
        orc.fwd(q, q, q, window=4, causal=False)
    except Exception as e:  # OracleError
        assert "returned -1" in str(e)
        return
    raise AssertionError("causal=False with a window must be rejected")


# ---------------------------------------------------------------- second implementation
BRUTE_SHAPES = [
    # B,Hq,Hkv,Q,K,D,Dv, window, seqlens
    (1, 4, 2, 5, 9, 8, 8, 0, None),
    (1, 4, 2, 9, 5, 8, 8, 0, None),            # more rows than keys
    (2, 2, 1, 3, 35, 7, 3, 0, None),           # odd widths
    (1, 2, 1, 3, 67, 33, 7, 4, None),
    (3, 4, 4, 4, 12, 16, 8, 3, [0, 12, 5]),
    (2, 8, 2, 1, 33, 16, 24, 0, [33, 1]),      # decode, MQA-like groups
]
# Non-causal and fp16-storage cases: B,Hq,Hkv,Q,K,D,Dv, seqlens, storage
BRUTE_EXTRA = [
    (1, 4, 2, 9, 5, 8, 8, None, "f32", False),
    (3, 4, 4, 4, 12, 16, 8, [0, 12, 5], "f32", False),
    (2, 4, 2, 6, 21, 16, 24, [21, 7], "f16", True),
    (1, 2, 1, 3, 35, 8, 8, None, "f16", False),
]


def pin_brute_force(orc):
    rng = np.random.default_rng(23)
    for (B, Hq, Hkv, Q, K, D, Dv, W, sl) in BRUTE_SHAPES:
        q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
        sla = None if sl is None else np.array(sl, np.int32)
        o, lse = orc.fwd(q, k, v, seqlens=sla, window=W)
        bo, bl = brute.attention(q, k, v, seqlens=sla, window=W)
        _close(o, bo, 1e-12, f"brute force O {B,Hq,Hkv,Q,K,D,Dv,W,sl}")
        _close(lse, bl, 1e-12, f"brute force LSE {B,Hq,Hkv,Q,K,D,Dv,W,sl}")
    for (B, Hq, Hkv, Q, K, D, Dv, sl, st, causal) in BRUTE_EXTRA:
        mk = (lambda shape: _f32(rng, shape).astype(np.float16)) if st == "f16" else (lambda shape: _f32(rng, shape))
        q, k, v = mk((B, Hq, Q, D)), mk((B, Hkv, K, D)), mk((B, Hkv, K, Dv))
        sla = None if sl is None else np.array(sl, np.int32)
        o, lse = orc.fwd(q, k, v, seqlens=sla, causal=causal)
        bo, bl = brute.attention(q, k, v, seqlens=sla, causal=causal)
        _close(o, bo, 1e-12, f"brute force O {B,Hq,Hkv,Q,K,D,Dv,sl,st,causal}")
        _close(lse, bl, 1e-12, f"brute force LSE {B,Hq,Hkv,Q,K,D,Dv,sl,st,causal}")


# ---------------------------------------------------------------------------
# Backward (gradients of sum(dO * O) w.r.t. q, k, v)
# ---------------------------------------------------------------------------

def _loss(orc, q, k, v, dout, **kw):
    o, _ = orc.fwd(q, k, v, **kw)
    return float(np.sum(dout * o))


def pin_bwd_finite_differences(orc):
    """Every gradient element against a central difference of the (pinned)
    fp64 forward: sum(dO * O(x + e)) - sum(dO * O(x - e)) over 2e, float64 inputs."""
    rng = np.random.default_rng(40)
    B, Hq, Hkv, Q, K, D, Dv = 2, 4, 2, 3, 6, 4, 3
    cases = [dict(seqlens=np.array([6, 2], np.int32)), dict(window=2), dict(causal=False, seqlens=np.array([4, 6], np.int32)),
             dict(scale=-0.7)]
    for kw in cases:
        q = rng.standard_normal((B, Hq, Q, D))
        k = rng.standard_normal((B, Hkv, K, D))
        v = rng.standard_normal((B, Hkv, K, Dv))
        dout = rng.standard_normal((B, Hq, Q, Dv))
        dq, dk, dv = orc.bwd(q, k, v, dout, **kw)
        eps = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for i in np.ndindex(x.shape):
                x0 = x[i]
                x[i] = x0 + eps
                lp = _loss(orc, q, k, v, dout, **kw)
                x[i] = x0 - eps
                lm = _loss(orc, q, k, v, dout, **kw)
                x[i] = x0
                num[i] = (lp - lm) / (2 * eps)
            _close(g, num, 1e-7, f"d{name} vs central differences {sorted(kw)}")


def _torch_attention(q, k, v, kb, window, causal, scale):
    """Plain masked attention in torch float64 (kv heads repeated over groups)."""
    B, Hq, Q, D = q.shape
    Hkv, K = k.shape[1], k.shape[2]
    g = Hq // Hkv
    ke = k.repeat_interleave(g, dim=1)
    ve = v.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(q, ke.transpose(-1, -2))
    kpos = torch.arange(K).view(1, K)
    outs = []
    for b in range(B):
        p = torch.arange(Q).view(Q, 1) + int(kb[b]) - Q
        m = kpos < int(kb[b])
        if causal:
            m = m & (kpos <= p)
        if window > 0:
            m = m & (kpos > p - window)
        sb = s[b].masked_fill(~m, float("-inf"))
        w = torch.softmax(sb, dim=-1)
        w = torch.nan_to_num(w, nan=0.0)  # rows with no legal key
        outs.append(torch.matmul(w, ve[b]))
    return torch.stack(outs)


def pin_bwd_torch_autograd(orc):
    """Gradients against torch autograd through plain masked attention in float64."""
    rng = np.random.default_rng(41)
    for (B, Hq, Hkv, Q, K, D, Dv), kw in [((2, 4, 2, 7, 9, 8, 6), dict(seqlens=[9, 3])),
                                           ((1, 6, 3, 5, 5, 16, 16), dict(window=3)),
                                           ((2, 4, 1, 4, 11, 8, 12), dict(causal=False, seqlens=[0, 11])),
                                           ((1, 2, 2, 12, 6, 4, 4), dict())]:
        q = rng.standard_normal((B, Hq, Q, D))
        k = rng.standard_normal((B, Hkv, K, D))
        v = rng.standard_normal((B, Hkv, K, Dv))
        dout = rng.standard_normal((B, Hq, Q, Dv))
        sl = kw.get("seqlens")
        scale = 1.0 / math.sqrt(D)
        okw = dict(window=kw.get("window", 0), causal=kw.get("causal", True))
        if sl is not None:
            okw["seqlens"] = np.array(sl, np.int32)
        dq, dk, dv = orc.bwd(q, k, v, dout, **okw)
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        kb = sl if sl is not None else [K] * B
        o = _torch_attention(tq, tk, tv, kb, okw["window"], okw["causal"], scale)
        gq, gk, gv = torch.autograd.grad((o * torch.from_numpy(dout)).sum(), (tq, tk, tv))
        what = f"{(B, Hq, Hkv, Q, K, D, Dv)} {kw}"
        _close(dq, gq.numpy(), 1e-10, "dq vs torch autograd " + what)
        _close(dk, gk.numpy(), 1e-10, "dk vs torch autograd " + what)
        _close(dv, gv.numpy(), 1e-10, "dv vs torch autograd " + what)


def pin_bwd_closed_forms(orc):
    """(a) window 1: every row sees one key (weight 1): dQ = dK = 0 and dV[k] is
    the sum of dO over the rows whose diagonal is k; (b) dO = 0: every gradient
    is 0; (c) identical keys: uniform weights, dQ = 0 and dV[k] = mean of dO."""
    rng = np.random.default_rng(42)
    B, Hq, Hkv, Q, K, D, Dv = 1, 4, 2, 5, 8, 8, 4
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    dout = _f32(rng, (B, Hq, Q, Dv))
    dq, dk, dv = orc.bwd(q, k, v, dout, window=1)
    _close(dq, np.zeros_like(dq), 1e-15, "window 1: dQ")
    _close(dk, np.zeros_like(dk), 1e-15, "window 1: dK")
    want = np.zeros_like(dv)
    g = Hq // Hkv
    for h in range(Hq):
        for qi in range(Q):
            want[0, h // g, qi + K - Q] += dout[0, h, qi]
    _close(dv, want, 1e-12, "window 1: dV")
    dq, dk, dv = orc.bwd(q, k, v, np.zeros_like(dout))
    for name, a in (("dq", dq), ("dk", dk), ("dv", dv)):
        _close(a, np.zeros_like(a), 0.0, f"dO = 0: {name}")
    kc = np.ascontiguousarray(np.repeat(k[:, :, :1], K, axis=2))
    dq, dk, dv = orc.bwd(q, kc, v, dout, causal=False)
    _close(dq, np.zeros_like(dq), 1e-12, "identical keys: dQ")
    want = np.zeros_like(dv)
    for h in range(Hq):
        want[0, h // g] += dout[0, h].astype(np.float64).sum(axis=0) / K
    _close(dv, want, 1e-12, "identical keys: dV")


def pin_bwd_gqa_sum(orc):
    """A kv-head's dK/dV is the sum over its query heads of the MHA gradients
    with K/V repeated; dQ is the same."""
    rng = np.random.default_rng(43)
    B, Hq, Hkv, Q, K, D, Dv = 2, 6, 2, 4, 9, 8, 8
    q, k, v = _f32(rng, (B, Hq, Q, D)), _f32(rng, (B, Hkv, K, D)), _f32(rng, (B, Hkv, K, Dv))
    dout = _f32(rng, (B, Hq, Q, Dv))
    sl = np.array([9, 5], np.int32)
    dq, dk, dv = orc.bwd(q, k, v, dout, seqlens=sl, window=4)
    g = Hq // Hkv
    ke, ve = np.ascontiguousarray(np.repeat(k, g, axis=1)), np.ascontiguousarray(np.repeat(v, g, axis=1))
    dq2, dk2, dv2 = orc.bwd(q, ke, ve, dout, seqlens=sl, window=4)
    _close(dq, dq2, 1e-12, "GQA dQ equals MHA dQ")
    _close(dk, dk2.reshape(B, Hkv, g, K, D).sum(axis=2), 1e-12, "GQA dK = sum of MHA dK over the group")
    _close(dv, dv2.reshape(B, Hkv, g, K, Dv).sum(axis=2), 1e-12, "GQA dV = sum of MHA dV over the group")


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_closed_forms, pin_bwd_gqa_sum]

INDEPENDENT_PINS = [
    pin_worked_examples, pin_textbook_causal, pin_bottom_right, pin_uniform_v, pin_single_key,
    pin_scale_zero, pin_empty_rows, pin_shift_invariance, pin_probs_sum_to_one, pin_split_merge,
    pin_gqa_expand, pin_varlen_unpadded, pin_v_columns_untouched, pin_fp16_decode, pin_noncausal_textbook,
    pin_noncausal_key_order, pin_noncausal_closed_forms, pin_noncausal_needs_no_window,
]
ALL_PINS = INDEPENDENT_PINS + BWD_PINS + [pin_brute_force]

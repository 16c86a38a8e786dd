"""Dense brute-force attention for tiny inputs -- TEST INFRASTRUCTURE ONLY.

A second, independent CPU implementation in pure Python/numpy: it builds the
whole [Q, K] boolean mask and score matrix for each (batch, head) and sums
with math.fsum (correctly rounded).  It exists to cross-check the C oracle on
small shapes; it follows the same definition (LuisaCompute "Attention
execution mapping" review, section 1; per-sequence lengths and window as read
in the design notes; causal=False drops the causal limit) but shares no code
with it.
"""
from __future__ import annotations

import math

import numpy as np


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16), float16 or float32 -> float64 (all exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def attention(q, k, v, *, seqlens=None, window=0, scale=None, causal=True):
    qd, kd, vd = widen(q), widen(k), widen(v)
    B, Hq, Q, D = qd.shape
    _, Hkv, K, _ = kd.shape
    Dv = vd.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    group = Hq // Hkv
    o = np.zeros((B, Hq, Q, Dv))
    lse = np.full((B, Hq, Q), -np.inf)
    for b in range(B):
        Kb = K if seqlens is None else int(seqlens[b])
        qpos = np.arange(Q)[:, None] + Kb - Q          # absolute position of each query row
        kpos = np.arange(K)[None, :]
        mask = (kpos < Kb) & np.ones((Q, 1), dtype=bool)
        if causal:
            mask &= kpos <= qpos
        if window > 0:
            mask &= kpos > qpos - window
        for h in range(Hq):
            kh = h // group
            s = scale * (qd[b, h] @ kd[b, kh].T)      # [Q, K]
            for i in range(Q):
                idx = np.nonzero(mask[i])[0]
                if len(idx) == 0:
                    continue
                row = s[i, idx]
                m = max(row)
                e = [math.exp(x - m) for x in row]
                tot = math.fsum(e)
                for j in range(Dv):
                    o[b, h, i, j] = math.fsum(e[t] / tot * vd[b, kh, idx[t], j] for t in range(len(idx)))
                lse[b, h, i] = m + math.log(tot)
    return o, lse

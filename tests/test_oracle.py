"""The fp64 oracle against its pins (CPU only).

The pins live in tests/pins.py; each is a check against something other than
the oracle itself: hand-worked examples, torch's textbook causal attention,
closed forms and invariants of the definition.
"""
import numpy as np
import pytest

import pins

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_sizes(orc):
    from oracle.attn_oracle import OracleError
    q = np.zeros((1, 3, 2, 4), np.float32)
    k = np.zeros((1, 2, 5, 4), np.float32)
    with pytest.raises(OracleError):
        orc.fwd(q, k, k)  # Hq % Hkv != 0
    q = np.zeros((1, 2, 2, 4), np.float32)
    with pytest.raises(OracleError):
        orc.fwd(q, k, k, seqlens=np.array([6], np.int32))  # length beyond K


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode", ["causal_window", "causal", "noncausal", "noncausal_empty"])
def test_oracle_rows_match_full(orc, dtype, mode):
    """The row-sampled oracle (used on the large workloads) is the full oracle's
    arithmetic row by row: bitwise the same rows, in every storage type and in
    both masking modes, with per-sequence lengths (one sequence empty in the
    last mode)."""
    from attention_attn_fwd_amd import inputs
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Q, K, D, Dv = 3, 4, 2, 7, 19, 16, 8
    qf = rng.standard_normal((B, Hq, Q, D)).astype(np.float32)
    kf = rng.standard_normal((B, Hkv, K, D)).astype(np.float32)
    vf = rng.standard_normal((B, Hkv, K, Dv)).astype(np.float32)
    conv = {"f32": lambda a: a, "f16": lambda a: a.astype(np.float16), "bf16": inputs.f32_to_bf16_bits}[dtype]
    q, k, v = conv(qf), conv(kf), conv(vf)
    sl = np.array([19, 4, 0 if mode == "noncausal_empty" else 11], np.int32)
    kw = {"causal_window": dict(seqlens=sl, window=5), "causal": dict(seqlens=sl),
          "noncausal": dict(seqlens=sl, causal=False), "noncausal_empty": dict(seqlens=sl, causal=False)}[mode]
    o, lse = orc.fwd(q, k, v, **kw)
    rows = np.arange(B * Hq * Q, dtype=np.int64)[::3]
    ro, rl = orc.rows(q, k, v, rows, **kw)
    np.testing.assert_array_equal(ro, o.reshape(-1, Dv)[rows])
    np.testing.assert_array_equal(rl, lse.reshape(-1)[rows])
    if mode == "noncausal_empty":  # the empty sequence's rows: O = 0, LSE = -inf
        sel = rows // (Hq * Q) == 2
        assert np.all(ro[sel] == 0.0) and np.all(np.isneginf(rl[sel]))


def test_oracle_bf16_inputs(orc):
    """bf16 bit patterns are widened exactly: same result as their float32 values."""
    from attention_attn_fwd_amd import inputs
    w = inputs.Workload("t", 1, 4, 2, 6, 13, 16, 16)
    q, k, v = w.gen_q(), w.gen_k(), w.gen_v()
    o1, l1 = orc.fwd(q, k, v)
    f = inputs.bf16_bits_to_f32
    o2, l2 = orc.fwd(f(q), f(k), f(v))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_oracle_bwd_samples_match_full(orc):
    """The sampled backward (dq of chosen rows, dk/dv of chosen keys) equals the
    full backward's entries."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, Q, K, D, Dv = 2, 6, 2, 9, 21, 16, 8
    q = rng.standard_normal((B, Hq, Q, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, K, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, K, Dv)).astype(np.float32)
    dout = rng.standard_normal((B, Hq, Q, Dv)).astype(np.float32)
    for kw in (dict(seqlens=np.array([21, 6], np.int32), window=5), dict(causal=False)):
        dq, dk, dv = orc.bwd(q, k, v, dout, **kw)
        rows = np.array([0, 4, 17, 50, 107], np.int64)
        np.testing.assert_allclose(orc.bwd_rows(q, k, v, dout, rows, **kw), dq.reshape(-1, D)[rows], rtol=0,
                                   atol=1e-12)
        keys = np.array([0, 3, 20, 22, 40, 83], np.int64)
        sk, sv = orc.bwd_keys(q, k, v, dout, keys, **kw)
        np.testing.assert_allclose(sk, dk.reshape(-1, D)[keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sv, dv.reshape(-1, Dv)[keys], rtol=0, atol=1e-12)

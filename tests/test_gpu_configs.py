"""The five benchmark workloads at full size, in the launch configuration the
bench times, compared with the fp64 oracle on every element: the two small
ones in one piece, the three large ones one sequence at a time (each
sequence of a batch is its own problem, so the oracle runs on the slice),
after one GPU run per configuration.  Whole-output properties are checked
as well: every row written, no NaN/Inf, LSE = -inf exactly on the rows
without a legal key, bitwise-identical reruns, inputs unchanged.
"""
import numpy as np
import pytest

from attention_attn_fwd_amd import inputs
from gpu_util import compare, run_gpu, say

pytestmark = pytest.mark.gpu


def _sample_rows(w, n, seed=0):
    """Flat row ids (b*Hq+h)*Q+q: tile edges, first/last rows, and random rows."""
    rng = np.random.default_rng(seed)
    qs = {0, w.Q - 1}
    for edge in (127, 128, 255, 256, w.Q // 2):
        if 0 <= edge < w.Q:
            qs.add(edge)
    rows = set()
    for b in range(w.B):
        for q in qs:
            rows.add((b * w.Hq + int(rng.integers(w.Hq))) * w.Q + q)
    while len(rows) < n:
        rows.add(int(rng.integers(w.B * w.Hq * w.Q)))
    return np.array(sorted(rows), dtype=np.int64)


def _empty_rows_mask(w):
    """True where a row has no legal key: q + K_b - Q < 0 (the window always keeps the diagonal)."""
    kb = np.array([w.kb(b) for b in range(w.B)])[:, None, None]
    q = np.arange(w.Q)[None, None, :]
    return np.broadcast_to(q + kb - w.Q < 0, (w.B, w.Hq, w.Q))


def _gpu_config(idx):
    """One GPU run of configuration idx with the whole-output checks; returns the
    workload, its host inputs and the GPU outputs (float64 host arrays)."""
    w = inputs.config(idx)
    say(f"[config {idx}] {w.name} {w.shape_tuple} {w.dtype} W={w.window}")
    q = w.gen_q()
    k = w.gen_k(padding="zero")
    v = w.gen_v(padding="zero")
    o, lse = run_gpu(w, q, k, v, check_inputs=(idx <= 4))
    empty = _empty_rows_mask(w)
    assert np.array_equal(np.isneginf(lse), empty), "LSE -inf pattern differs from the rows without keys"
    assert np.all(o[empty] == 0.0)
    assert np.isfinite(o).all() and not np.isnan(lse).any()
    return w, q, k, v, o, lse


def _compare_sequence(run, orc, b):
    """Every element of sequence b against the oracle run on that sequence alone."""
    w, q, k, v, o, lse = run
    sl = None if w.seqlens is None else w.seqlens[b:b + 1]
    say(f"[config] {w.name} sequence {b} (K_b = {w.kb(b)}): full oracle")
    ro, rl = orc.fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], seqlens=sl, window=w.window, scale=w.scale)
    return compare(o[b:b + 1], lse[b:b + 1], ro, rl, w.dtype, f"{w.name} sequence {b}")


@pytest.fixture(scope="module")
def run3():
    return _gpu_config(3)


@pytest.fixture(scope="module")
def run4():
    return _gpu_config(4)


@pytest.fixture(scope="module")
def run5():
    return _gpu_config(5)


def test_config1_tiny_fp32(orc):
    w, q, k, v, o, lse = _gpu_config(1)
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale)
    compare(o, lse, ro, rl, w.dtype, w.name)


def test_config2_decode_tail(orc):
    w, q, k, v, o, lse = _gpu_config(2)
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale)
    compare(o, lse, ro, rl, w.dtype, w.name)


@pytest.mark.parametrize("b", range(4))
def test_config3_dense_prefill_full(orc, run3, b):
    _compare_sequence(run3, orc, b)


@pytest.mark.parametrize("b", range(16))
def test_config4_varlen_window_full(orc, run4, b):
    _compare_sequence(run4, orc, b)


def test_config5_long_decode_full(orc, run5):
    w, q, k, v, o, lse = run5
    say(f"[config] {w.name}: full oracle over all {w.B} sequences")
    ro, rl = orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale)
    compare(o, lse, ro, rl, w.dtype, w.name)


# The option workloads the bench times beside the step, at their full sizes,
# on sampled rows: fp16 storage and the non-causal mode at the dense prefill
# shape, heads of 256 and 512 channels there, the two chunked-prefill shapes
# (packed tiles and split key ranges), fp16 storage at the long decode shape.
def _run_option(w, orc, n_rows):
    import dataclasses  # noqa: F401
    say(f"[option] {w.name} {w.shape_tuple} {w.dtype} causal={w.causal} W={w.window}")
    q = w.gen_q()
    k = w.gen_k(padding="zero")
    v = w.gen_v(padding="zero")
    o, lse = run_gpu(w, q, k, v, check_inputs=False)
    assert np.isfinite(o).all() and not np.isnan(lse).any()
    rows = _sample_rows(w, n_rows)
    ro, rl = orc.rows(q, k, v, rows, seqlens=w.seqlens, window=w.window, scale=w.scale, causal=w.causal)
    return compare(o.reshape(-1, w.Dv)[rows], lse.reshape(-1)[rows], ro, rl, w.dtype, f"{w.name} ({len(rows)} rows)")


def _c3(**kw):
    import dataclasses
    return dataclasses.replace(inputs.config(3), **kw)


@pytest.mark.parametrize("variant", ["f16", "noncausal", "d256", "d512"])
def test_option_dense_prefill_shape(orc, variant):
    kw = {"f16": dict(name="c3_shape_f16", dtype="f16"), "noncausal": dict(name="c3_shape_noncausal", causal=False),
          "d256": dict(name="c3_shape_d256", D=256, Dv=256), "d512": dict(name="c3_shape_d512", D=512, Dv=512)}
    _run_option(_c3(**kw[variant]), orc, 256)


@pytest.mark.parametrize("shape", [(4, 32, 8, 64, 16384, 128, 128), (1, 32, 8, 512, 32768, 128, 128)],
                         ids=["chunk64_ctx16k", "chunk512_ctx32k"])
def test_option_chunked_prefill(orc, shape):
    _run_option(inputs.Workload("chunk", *shape), orc, 256)


def test_option_long_decode_f16(orc):
    import dataclasses
    _run_option(dataclasses.replace(inputs.config(5), name="c5_shape_f16", dtype="f16"), orc, 512)

"""The seeded input generator (CPU): Philox known answers, Box-Muller, bf16 rounding, recipes."""
import math

import numpy as np
import pytest

from attention_attn_fwd_amd import inputs


def test_philox_known_answers():
    # Known-answer vectors of Philox-4x32-10 published with the Random123 reference
    # implementation (Salmon et al., SC'11): counter, key -> output words.
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
        ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
        ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
         [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
    ]
    for ctr, key, want in kat:
        assert inputs.philox4x32_10(ctr, key) == want


def test_box_muller_radius():
    """Elements 4j and 4j+1 share (u1, u2): z0^2 + z1^2 = -2 ln u1 with u1 from word 0."""
    n = 4096
    z = inputs.normal((n,), tensor_id=7, seed=99, dtype="f32").astype(np.float64)
    w = inputs.uniform_words(n, tensor_id=7, seed=99)
    u1 = (w[0::4].astype(np.float64) + 0.5) / 2 ** 32
    r2 = z[0::4] ** 2 + z[1::4] ** 2
    np.testing.assert_allclose(r2, -2.0 * np.log(u1), rtol=2e-6, atol=1e-6)
    u1b = (w[2::4].astype(np.float64) + 0.5) / 2 ** 32
    np.testing.assert_allclose(z[2::4] ** 2 + z[3::4] ** 2, -2.0 * np.log(u1b), rtol=2e-6, atol=1e-6)


def test_normal_moments():
    z = inputs.normal((1 << 20,), tensor_id=1, dtype="f32").astype(np.float64)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert abs(np.mean(np.abs(z) < 1.0) - 0.682689492) < 5 * math.sqrt(0.25 / n)
    assert abs(np.mean(z ** 4) - 3.0) < 0.05


def test_slices_regenerate_exactly():
    full = inputs.normal((3, 5, 7, 16), tensor_id=2)
    part = inputs.normal((2, 16), tensor_id=2, offset=((1 * 5 + 3) * 7 + 4) * 16)
    np.testing.assert_array_equal(part, full[1, 3, 4:6])
    w = inputs.Workload("t", 3, 5, 5, 7, 9, 16, 16)
    np.testing.assert_array_equal(w.gen_rows("q", 1, 3, 4, 6), w.gen_q()[1, 3, 4:6])
    np.testing.assert_array_equal(w.gen_rows("v", 2, 4, 0, 9), w.gen_v()[2, 4])


def test_deterministic_and_thread_independent():
    a = inputs.normal((100003,), tensor_id=3, threads=1)
    b = inputs.normal((100003,), tensor_id=3, threads=8)
    np.testing.assert_array_equal(a, b)
    c = inputs.normal((100003,), tensor_id=3, seed=1235)
    assert not np.array_equal(a, c)


def test_bf16_round_to_nearest_even():
    """Check the rounding against its definition: nearest bf16 value, ties to an even mantissa."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    r = inputs.f32_to_bf16_bits(x)
    rf = inputs.bf16_bits_to_f32(r).astype(np.float64)
    xd = x.astype(np.float64)
    lo_bits = (x.view(np.uint32) & 0xFFFF0000).astype(np.uint32)
    lo = lo_bits.view(np.float32).astype(np.float64)            # truncation toward zero
    hi = (lo_bits + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
    d_r = np.abs(rf - xd)
    assert np.all(d_r <= np.minimum(np.abs(lo - xd), np.abs(hi - xd)) + 0.0)
    ties = np.abs(lo - xd) == np.abs(hi - xd)
    assert np.all((r[ties] & 1) == 0)
    # explicit ties and specials
    cases = {0x3F808000: 0x3F80, 0x3F818000: 0x3F82, 0x3F80C000: 0x3F81, 0x7F7FFFFF: 0x7F80,
             0x00000000: 0x0000, 0x80000000: 0x8000}
    xs = np.array(list(cases), dtype=np.uint32).view(np.float32)
    np.testing.assert_array_equal(inputs.f32_to_bf16_bits(xs), np.array(list(cases.values()), np.uint16))
    nan = inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(inputs.bf16_bits_to_f32(nan))[0]


def test_bf16_stream_is_rounded_f32_stream():
    f = inputs.normal((4099,), tensor_id=5, dtype="f32")
    b = inputs.normal((4099,), tensor_id=5, dtype="bf16")
    np.testing.assert_array_equal(inputs.f32_to_bf16_bits(f), b)


def test_f16_stream_is_rounded_f32_stream():
    f = inputs.normal((4099,), tensor_id=5, dtype="f32")
    h = inputs.normal((4099,), tensor_id=5, dtype="f16")
    assert h.dtype == np.float16
    np.testing.assert_array_equal(f.astype(np.float16), h)
    # round to nearest, ties to even: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    ties = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11], dtype=np.float32)
    np.testing.assert_array_equal(ties.astype(np.float16).astype(np.float64), [1.0, 1.0 + 2 * 2.0 ** -10])
    part = inputs.normal((7,), tensor_id=5, dtype="f16", offset=100)
    np.testing.assert_array_equal(part, h[100:107])


def test_noncausal_pair_count():
    w = inputs.Workload("nc", 2, 4, 2, 5, 9, 16, 16, causal=False, seqlens=np.array([9, 3], np.int32))
    assert w.legal_pairs() == 4 * 5 * (9 + 3)


def test_config_recipes():
    c1 = inputs.config(1)
    assert c1.shape_tuple == (1, 4, 2, 64, 128, 64, 64) and c1.dtype == "f32" and c1.seqlens is None
    assert c1.legal_pairs() == 24704
    c2 = inputs.config(2)
    assert c2.shape_tuple == (1, 8, 2, 1, 2053, 80, 96) and c2.legal_pairs() == 8 * 2053
    c3 = inputs.config(3)
    assert c3.shape_tuple == (4, 32, 8, 4096, 4096, 128, 128) and c3.legal_pairs() == 1074003968
    c4 = inputs.config(4)
    assert c4.window == 1024 and c4.seqlens.dtype == np.int32
    assert c4.seqlens[1] == 0 and c4.seqlens[14] == 0
    assert np.all((c4.seqlens >= 0) & (c4.seqlens <= 4096))
    np.testing.assert_array_equal(c4.seqlens, inputs.config(4).seqlens)
    c5 = inputs.config(5)
    assert np.all((c5.seqlens >= 1024) & (c5.seqlens <= 32768))
    # log-uniform: the median of log2(len) sits near the middle of [10, 15]
    assert 11.5 < np.median(np.log2(c5.seqlens)) < 13.5


def test_seqlens_uniform_covers_range():
    s = inputs.seqlens_uniform(20000, 4096, seed=7)
    assert s.min() >= 0 and s.max() <= 4096
    assert abs(s.mean() - 2048) < 40


def test_zero_padding_keeps_valid_rows():
    w = inputs.Workload("t", 3, 4, 2, 2, 37, 16, 32, seqlens=np.array([37, 0, 11], np.int32))
    full, lean = w.gen_k(), w.gen_k(padding="zero")
    for b in range(3):
        kb = w.kb(b)
        np.testing.assert_array_equal(lean[b, :, :kb], full[b, :, :kb])
        assert not lean[b, :, kb:].any()
    np.testing.assert_array_equal(w.gen_v(padding="zero")[2, :, :11], w.gen_v()[2, :, :11])

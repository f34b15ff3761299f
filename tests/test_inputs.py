"""The seeded input generator: determinism, rounding, and the workload recipes (no GPU)."""

import numpy as np
import pytest

import fa2_inputs as gen
from oracle import bf16_bits_to_float64


def test_rne_rounding_ties_and_specials():
    words = np.array([
        0x3F800000,  # 1.0 exactly
        0x3F808000,  # halfway, lower kept bit even -> down to 0x3F80
        0x3F818000,  # halfway, lower kept bit odd  -> up to 0x3F82
        0x3F808001,  # just above halfway -> up
        0x3F807FFF,  # just below halfway -> down
        0x7F7FFFFF,  # largest float32 -> rounds to +inf in bf16
        0xFF800000,  # -inf
        0x00000001,  # tiny denormal -> +0
    ], dtype=np.uint32)
    got = gen.round_to_bf16_bits(words.view(np.float32))
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80, 0x7F80, 0xFF80, 0x0000]
    nan = gen.round_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_float64(nan)[0])


def test_rounding_error_is_at_most_half_ulp():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    r = bf16_bits_to_float64(gen.round_to_bf16_bits(x))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x.astype(np.float64)))) - 7)
    assert np.all(np.abs(r - x) <= ulp / 2)


def test_deterministic_and_seed_dependent():
    a = gen.make_arrays(2, 3, 40, 16, seed=5)
    b = gen.make_arrays(2, 3, 40, 16, seed=5)
    c = gen.make_arrays(2, 3, 40, 16, seed=6)
    for key in ("q", "k", "v", "do"):
        assert a[key].dtype == np.uint16 and a[key].shape == (2, 3, 40, 16)
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    assert not np.array_equal(a["q"], a["k"])


def test_spike_rows_are_exact_x8_and_sigma():
    plain = gen.make_arrays(2, 4, 64, 80, seed=3, sigma=0.5, spike=False)
    spiky = gen.make_arrays(2, 4, 64, 80, seed=3, sigma=0.5, spike=True)
    rows = spiky["spike_rows"]
    assert rows.shape == (2, 4)
    for name in ("q", "k"):
        p = bf16_bits_to_float64(plain[name])
        s = bf16_bits_to_float64(spiky[name])
        for b in range(2):
            for h in range(4):
                r = rows[b, h]
                np.testing.assert_array_equal(s[b, h, r], 8.0 * p[b, h, r])
                mask = np.ones(64, bool)
                mask[r] = False
                np.testing.assert_array_equal(s[b, h, mask], p[b, h, mask])
    for name in ("v", "do"):
        assert np.array_equal(plain[name], spiky[name])
    std = bf16_bits_to_float64(plain["v"]).std()
    assert std == pytest.approx(0.5, rel=0.02)


def test_workload_table():
    w = gen.WORKLOADS
    assert [(x.B, x.H, x.N, x.d, x.causal) for x in w.values()] == [
        (1, 1, 128, 64, False), (8, 16, 2048, 128, False), (4, 32, 4096, 64, True),
        (1, 16, 16384, 128, True), (2, 32, 8192, 80, True)]
    assert w["c5"].sigma == 0.5 and w["c5"].spike
    assert w["c1"].scale == np.float32(0.125)
    # conventional flop counts: 4 B H N^2 d forward, x2.5 backward, halved when causal
    assert w["c2"].flops("fwd") == 4 * 8 * 16 * 2048 ** 2 * 128
    assert w["c4"].flops("fwdbwd") == pytest.approx(3.8483e12, rel=1e-4)


def test_fp16_rounding_is_nearest_even():
    one = 1.0
    x = np.array([one, one + 2.0 ** -11, one + 3 * 2.0 ** -11, -2.5, 65504.0, 65520.0, 2.0 ** -25 * 3],
                 dtype=np.float32)
    got = gen.round_to_fp16_bits(x)
    # 1 + 2^-11 is halfway: to 1.0 (even); 1 + 3*2^-11 halfway: to 1 + 2^-9 (even);
    # 65520 is halfway to the overflow threshold: to infinity; 1.5 * 2^-24 -> 2^-23 (even)
    assert got.tolist() == [0x3C00, 0x3C00, 0x3C02, 0xC100, 0x7BFF, 0x7C00, 0x0002]


def test_fp16_arrays_match_bf16_draws():
    a16 = gen.make_arrays(1, 2, 40, 64, seed=9, dtype="fp16")
    ab = gen.make_arrays(1, 2, 40, 64, seed=9)
    for n in ("q", "k", "v", "do"):
        f = a16[n].view(np.float16).astype(np.float64)
        b = (ab[n].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        # the same draws, rounded to two formats: within one bf16 half-ulp of each other
        assert np.all(np.abs(f - b) <= np.abs(b) * 2.0 ** -8 + 1e-7)

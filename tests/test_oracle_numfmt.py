"""Pins for the oracle's number-format conversions (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def test_bf16_matches_torch_on_float32_values():
    # torch's float32 -> bfloat16 cast rounds to nearest even; on values that
    # are exactly float32 the oracle's fp64 -> bf16 must give the same bits.
    g = np.random.default_rng(0)
    x32 = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (g.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_ties_and_no_double_rounding():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2.0 ** -8: 0x3F80,                 # tie -> even (mantissa 0)
        one + 3 * 2.0 ** -8: 0x3F82,             # tie -> even (mantissa 2)
        one + 2.0 ** -8 + 2.0 ** -40: 0x3F81,    # above the tie: rounds up
        -(one + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** -133: 0x0001,                     # smallest subnormal
        float(np.inf): 0x7F80,
    }
    for x, bits in cases.items():
        assert int(oracle.f64_to_bf16_bits(np.array([x]))[0]) == bits, x
    # a value whose float32 rounding lands on the tie: direct rounding differs
    x = one + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(x) == np.float32(one + 2.0 ** -8)


def test_bf16_round_trip_exact():
    b = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(b)), b)


def test_f16_rounding():
    cases = {1.0: 0x3C00, 1 + 2.0 ** -11: 0x3C00, 1 + 3 * 2.0 ** -11: 0x3C02,
             1 + 2.0 ** -11 + 2.0 ** -30: 0x3C01, 65504.0: 0x7BFF, 2.0 ** -24: 0x0001}
    for x, bits in cases.items():
        assert int(oracle.f64_to_f16_bits(np.array([x]))[0]) == bits, x
    b = np.arange(0, 0x7C00, 3, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_f16_bits(oracle.f16_bits_to_f64(b)), b)

"""Pins for the oracle's bfloat16 conversions (oracle/bf16.py) against torch's
own bfloat16 type and against closed-form rounding cases."""
import numpy as np
import torch

from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16


def test_widening_matches_torch_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_narrowing_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 1, 200000), rng.normal(0, 1e-30, 10000), rng.normal(0, 1e30, 10000),
        rng.normal(0, 1e-39, 1000),                       # float32 subnormal range
    ]).astype(np.float32)
    # exact ties: odd multiples of half a bf16 spacing
    ties = (np.arange(1, 2000, 2, dtype=np.float32) * np.float32(2.0 ** -8) + 1.0).astype(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([3.4e38, -3.4e38, 0.0, -0.0])])
    ours = f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_no_double_rounding_through_float32():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint between 1 and 1 + 2^-7.
    # Through float32 it would become the exact midpoint and round to even (1.0).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert round_to_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie -> even
    assert round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_overflow_and_special_values():
    big = float.fromhex("0x1.ff00000000000p+127")   # halfway above the largest bf16
    assert np.isinf(round_to_bf16(np.array([big]))[0])
    assert round_to_bf16(np.array([np.inf]))[0] == np.inf
    assert np.isnan(round_to_bf16(np.array([np.nan]))[0])
    assert round_to_bf16(np.array([2.0 ** -133]))[0] == 2.0 ** -133     # smallest subnormal
    assert round_to_bf16(np.array([2.0 ** -134]))[0] == 0.0             # tie -> even (zero)

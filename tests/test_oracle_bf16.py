"""bf16 rounding of the oracle against torch's conversion and hand-worked values."""

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16


def _torch_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_rne_on_random_and_ties():
    rng = np.random.default_rng(0)
    mant = rng.integers(0, 2**23, size=200_000, dtype=np.uint32)
    exp = rng.integers(1, 254, size=mant.size, dtype=np.uint32)
    sign = rng.integers(0, 2, size=mant.size, dtype=np.uint32)
    bits = (sign << 31) | (exp << 23) | mant
    ties = (bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)  # exactly halfway between two bf16 values
    sub = rng.integers(0, 2**23, size=20_000, dtype=np.uint32)  # fp32 subnormals
    allbits = np.concatenate([bits, ties, sub, sub | np.uint32(0x80000000)])
    x = allbits.view(np.float32)
    finite = np.isfinite(x) & (np.abs(x.astype(np.float64)) < 3.38e38)
    x = x[finite]
    np.testing.assert_array_equal(f64_to_bf16_bits(x), _torch_bits(x))


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0**-8, 0x3F80),            # tie between 1 and 1+2^-7: even mantissa (1) wins
    (1.0 + 3 * 2.0**-8, 0x3F82),        # tie between 1+2^-7 (odd) and 1+2^-6 (even)
    (1.0 + 2.0**-8 + 2.0**-30, 0x3F81),  # just above the tie rounds up
    (-(1.0 + 2.0**-8), 0xBF80),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0**-133, 0x0001),                # smallest bf16 subnormal
    (2.0**-134, 0x0000),                # half of it: tie to even (zero)
    (3 * 2.0**-134, 0x0002),            # tie between 1 and 2 quanta: even (2)
    (2.0**-126, 0x0080),                # smallest normal
    ((2 - 2.0**-7) * 2.0**127, 0x7F7F),  # largest finite
    ((2 - 2.0**-8) * 2.0**127, 0x7F80),  # tie above the largest finite rounds to inf
])
def test_hand_worked_values(value, bits):
    assert int(f64_to_bf16_bits(np.array([value]))[0]) == bits


def test_widening_round_trips_every_finite_pattern():
    b = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(b)
    fin = np.isfinite(v)
    np.testing.assert_array_equal(f64_to_bf16_bits(v[fin]), b[fin])
    np.testing.assert_array_equal(round_to_bf16(v[fin]), v[fin])


def test_non_finite_is_rejected():
    with pytest.raises(FloatingPointError):
        round_to_bf16(np.array([np.nan]))

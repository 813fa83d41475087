"""CPU checks of the bound the multi-projection GPU tests use to compare two results of
one computation whose fp32 sums were grouped differently
(gpu_util.assert_same_to_rounding): it admits what regrouping can do and rejects what
a wrong row, column or projection does."""

import numpy as np
import pytest

from gpu_util import assert_same_to_rounding


def _bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _next_away(bits):
    return ((bits & 0x8000) | ((bits & 0x7FFF) + 1)).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_admits_one_unit_flips(dtype):
    rng = np.random.default_rng(1)
    y = rng.standard_normal(20000).astype(np.float32)
    bits = _bf16_bits(y) if dtype == "bf16" else y.astype(np.float16).view(np.uint16)
    moved = bits.copy()
    moved[::5] = _next_away(moved[::5])
    assert_same_to_rounding(moved, bits, dtype)
    assert_same_to_rounding(bits, bits, dtype)


def test_admits_small_shift_near_zero():
    """A 2e-5 shift (a v entry rounded the other way) is many units of an output near 0."""
    y = np.array([1e-4, -3e-5, 0.5, 2.0], dtype=np.float32)
    a, b = _bf16_bits(y), _bf16_bits(y + np.float32(2e-5))
    assert not np.array_equal(a, b)
    assert_same_to_rounding(b, a, "bf16")


@pytest.mark.parametrize("shift", [5e-2, 2e-2])
def test_rejects_a_lora_sized_error(shift):
    rng = np.random.default_rng(2)
    y = rng.standard_normal(4096).astype(np.float32)
    bad = y.copy()
    bad[123] += np.float32(shift)
    with pytest.raises(AssertionError):
        assert_same_to_rounding(_bf16_bits(bad), _bf16_bits(y), "bf16")


def test_rejects_two_unit_flip_on_the_largest_element():
    y = np.array([3.9, 0.1, -1.0], dtype=np.float32)
    bits = _bf16_bits(y)
    two = bits.copy()
    two[0] = _next_away(_next_away(two[:1]))[0]
    with pytest.raises(AssertionError):
        assert_same_to_rounding(two, bits, "bf16")

"""Pins for the oracle's binary32/binary16 primitives (IEEE 754 facts, worked by hand)."""
import numpy as np
import pytest

from oracle.numerics import bf16_to_f32, to_f16, tree_sum
from synth import bf16_bits


def _f16_bits(x):
    return int(to_f16(np.float32(x)).view(np.uint16))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00),
    (1.0 + 2.0 ** -11, 0x3C00),            # exactly halfway 1.0 | 1+2^-10: ties to the even 0x3C00
    (1.0 + 3 * 2.0 ** -11, 0x3C02),        # halfway 0x3C01 | 0x3C02: ties to even 0x3C02
    (1.0 + 2.0 ** -11 + 2.0 ** -20, 0x3C01),  # just above halfway rounds up
    (2.0 ** -24, 0x0001),                  # smallest subnormal
    (2.0 ** -25, 0x0000),                  # halfway 0 | 2^-24: ties to even 0
    (3 * 2.0 ** -25, 0x0002),              # halfway 2^-24 | 2^-23: ties to even 2^-23
    (65504.0, 0x7BFF),                     # largest finite
    (65520.0, 0x7C00),                     # halfway 65504 | 65536: ties to even -> overflow to inf
    (-0.0, 0x8000),
    (1.0 / 127.0, 0x2008),                 # 2^-7 * (1 + 8.06/1024) -> mantissa 8
])
def test_f16_round_to_nearest_even(x, bits):
    assert _f16_bits(x) == bits


def test_bf16_widening_exact():
    b = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000], np.uint16)
    f = bf16_to_f32(b)
    assert f[0] == 1.0 and f[1] == -2.0
    assert f[2] == np.float32(2.0 ** -133)
    assert f[3] == np.float32(3.3895313892515355e38)
    assert np.signbit(f[4]) and f[4] == 0


def test_bf16_rounding_of_inputs_is_rne():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to even (1.0)
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    assert list(bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81]
    assert np.array_equal(bf16_to_f32(bf16_bits(x)), np.array([1, 1, 1 + 2 ** -6, 1 + 2 ** -7], np.float32))


def test_tree_sum_order():
    # Pairwise halving: (1e8 + -1e8) + (1 + 1) = 2, whereas a left-to-right binary32 sum gives 1.
    x = np.array([1e8, 1.0, -1e8, 1.0], np.float32)
    assert tree_sum(x) == np.float32(2.0)
    seq = np.float32(0)
    for v in x:
        seq = np.float32(seq + v)
    assert seq == np.float32(1.0)


def test_tree_sum_exact_on_integers():
    rng = np.random.default_rng(0)
    x = rng.integers(-1000, 1000, size=(7, 128)).astype(np.float32)
    assert np.array_equal(tree_sum(x), x.sum(axis=-1).astype(np.float32))
    with pytest.raises(ValueError):
        tree_sum(np.ones(6, np.float32))

"""Test helpers that decide pass / fail, checked on the CPU."""

import numpy as np

import oracle
from tests.gpu_util import bf16_ulp_distance


def test_bf16_ulp_distance_counts_representable_steps():
    # neighbours, zeros of both signs, and steps across zero
    a = np.array([0x3F80, 0x3F81, 0x0000, 0x8000, 0x8001, 0x0001, 0xBF80], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F80, 0x8000, 0x0001, 0x0001, 0x8001, 0xBF81], dtype=np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [1, 1, 0, 1, 2, 2, 1]
    # agrees with counting the bf16 values between two numbers
    rng = np.random.default_rng(0)
    x = rng.standard_normal(2000)
    y = x * (1 + 2.0 ** -7 * rng.integers(-3, 4, size=x.size))
    xb, yb = oracle.f64_to_bf16_bits(x), oracle.f64_to_bf16_bits(y)
    xs, ys = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(yb)
    grid = np.sort(oracle.bf16_bits_to_f64(np.arange(0, 0x7F80, dtype=np.uint16)))
    grid = np.concatenate([-grid[::-1], grid[1:]])   # every finite bf16 value once
    idx = lambda v: np.searchsorted(grid, v)
    assert np.array_equal(bf16_ulp_distance(xb, yb), np.abs(idx(xs) - idx(ys)))

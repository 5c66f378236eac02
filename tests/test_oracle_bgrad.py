"""Pins for the oracle's bias gradient (column sums of a bf16 matrix).

* exact summation: math.fsum (Shewchuk's exact algorithm, correctly rounded)
  per column on random data with a wide dynamic range;
* integer-valued columns: the sum equals Python integer arithmetic exactly;
* cancellation: columns made of +a / -a pairs sum to exactly zero;
* axis: a single non-zero element (r, c) lands in output c only, for every
  (r, c) of a small non-square matrix (catches a transposed reduction);
* signs and zero rows.
"""

import math

import numpy as np
import pytest

from oracle.bgrad import column_abs_sums, column_sums
from oracle.formats import bf16_to_float64


def bf16_bits(values) -> np.ndarray:
    """float values that are exactly representable in bf16 -> uint16 bit patterns."""
    f32 = np.asarray(values, dtype=np.float32)
    bits = f32.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def test_matches_exact_summation_wide_range():
    rng = np.random.default_rng(11)
    rows, cols = 300, 17
    mant = rng.integers(-255, 256, size=(rows, cols))
    expo = rng.integers(-40, 41, size=(rows, cols))
    vals = mant.astype(np.float64) * np.exp2(expo.astype(np.float64) - 8)
    bits = bf16_bits(vals)
    got = column_sums(bits)
    x = bf16_to_float64(bits)
    for c in range(cols):
        exact = math.fsum(x[:, c])
        bound = rows * 2.0 ** -53 * np.abs(x[:, c]).sum()
        assert abs(got[c] - exact) <= bound


def test_integer_columns_are_exact():
    rng = np.random.default_rng(12)
    ints = rng.integers(-128, 129, size=(1000, 9))
    got = column_sums(bf16_bits(ints))
    for c in range(9):
        assert got[c] == sum(int(v) for v in ints[:, c])


def test_cancelling_pairs_sum_to_zero():
    rng = np.random.default_rng(13)
    half = rng.integers(-255, 256, size=(64, 5)).astype(np.float64) * np.exp2(rng.integers(-20, 20, size=(64, 5)))
    vals = np.concatenate([half, -half[::-1]], axis=0)
    got = column_sums(bf16_bits(vals))
    assert np.all(got == 0.0)


def test_axis_single_element():
    rows, cols = 5, 3
    for r in range(rows):
        for c in range(cols):
            vals = np.zeros((rows, cols))
            vals[r, c] = -1.5 * 2.0 ** (r - c)
            got = column_sums(bf16_bits(vals))
            want = np.zeros(cols)
            want[c] = vals[r, c]
            assert np.array_equal(got, want)


def test_signs_zero_rows_and_abs_sums():
    vals = np.array([[1.0, -2.0, 0.0], [3.0, -4.0, -0.0], [-0.5, 8.0, 0.0]])
    bits = bf16_bits(vals)
    assert np.array_equal(column_sums(bits), np.array([3.5, 2.0, 0.0]))
    assert np.array_equal(column_abs_sums(bits), np.array([4.5, 14.0, 0.0]))
    empty = np.zeros((0, 4), np.uint16)
    assert np.array_equal(column_sums(empty), np.zeros(4))
    assert np.array_equal(column_abs_sums(empty), np.zeros(4))


def test_rejects_non_matrix():
    with pytest.raises(ValueError):
        column_sums(np.zeros(8, np.uint16))

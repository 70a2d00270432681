"""The bf16 comparison rule on hand-made values (CPU): one unit in the last
place from the oracle's correctly rounded value is accepted, and, given the
oracle's unrounded value, only when the two bf16 values bracket it."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle.compare import compare_bf16  # noqa: E402

ONE, NEXT, PREV = 0x3F80, 0x3F81, 0x3F7F      # 1.0, 1 + 2^-7, 1 - 2^-8


def b(*v):
    return np.array(v, np.uint16)


def test_identical_values_pass_with_their_rounding_error():
    r = compare_bf16(b(ONE), b(ONE), exact=np.array([1.0 + 2.0 ** -9]))
    assert r.n_diff == 0 and r.max_rel_exact == pytest.approx(2.0 ** -9 / (1 + 2.0 ** -9))


def test_one_unit_on_the_far_side_of_the_exact_value_passes():
    # exact 1 + 2^-8 - 2^-24 (just below the midpoint) rounds to 1.0; its other
    # neighbour is 1 + 2^-7
    r = compare_bf16(b(NEXT), b(ONE), exact=np.array([1.0 + 2.0 ** -8 - 2.0 ** -24]))
    assert r.n_diff == 1 and r.max_ulp == 1
    assert r.max_rel == pytest.approx(2.0 ** -7)             # 1 ulp of the rounded value
    assert r.max_rel_exact < 2.0 ** -8 + 2.0 ** -16          # half a unit of the exact value


def test_one_unit_on_the_near_side_fails_given_the_exact_value():
    with pytest.raises(AssertionError, match="bracket"):
        compare_bf16(b(PREV), b(ONE), exact=np.array([1.0 + 2.0 ** -9]))
    compare_bf16(b(PREV), b(ONE))                             # the ulp rule alone accepts it


def test_two_units_fail():
    with pytest.raises(AssertionError, match="ulp"):
        compare_bf16(b(0x3F82), b(ONE))


def test_signed_zeros_are_one_point_and_nan_must_match():
    assert compare_bf16(b(0x8000), b(0x0000), max_ulp=0).n_diff == 0
    with pytest.raises(AssertionError, match="NaN"):
        compare_bf16(b(0x7FC0), b(ONE))


def test_negative_values_bracket_the_same_way():
    # -(1 + 2^-8 - 2^-24) rounds to -1.0; the other neighbour is -(1 + 2^-7)
    compare_bf16(b(0x8000 | NEXT), b(0x8000 | ONE), exact=np.array([-(1.0 + 2.0 ** -8 - 2.0 ** -24)]))
    with pytest.raises(AssertionError, match="bracket"):
        compare_bf16(b(0x8000 | PREV), b(0x8000 | ONE), exact=np.array([-(1.0 + 2.0 ** -9)]))


def test_relative_error_to_the_exact_value_is_bounded_by_half_a_unit():
    # a value one unit off is accepted only next to a midpoint: 1 + 2^-8 - 2^-20
    # lies just below the midpoint of 1.0 and 1 + 2^-7, so either neighbour is
    # within 2^-8 (plus the allowance) of it
    compare_bf16(b(NEXT), b(ONE), exact=np.array([1.0 + 2.0 ** -8 - 2.0 ** -20]))
    # 1 + 2^-9 is a quarter unit above 1.0: its far neighbour is 3/4 unit away
    with pytest.raises(AssertionError, match="from the exact value"):
        compare_bf16(b(NEXT), b(ONE), exact=np.array([1.0 + 2.0 ** -9]))

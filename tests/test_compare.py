"""Pins of ``oracle.compare``, the function behind every parity assertion.

Each case is small enough to work out by hand; the expected figures are
written as the arithmetic that gives them, not as a call of the function.
A plausible slip in ``compare`` fails at least one case: normalising by the
norm of ``got`` instead of ``ref``, masking on ``got`` instead of ``ref``,
dropping the non-finite count, taking the mean instead of the maximum, or
losing the zero-norm branch.
"""
import math

import numpy as np

import oracle


def test_exact_match_is_zero():
    m = oracle.compare(np.array([1.5, -2.0, 0.25]), np.array([1.5, -2.0, 0.25]))
    assert m == {"max_abs": 0.0, "rel_l2": 0.0, "nonfinite": 0}


def test_max_abs_and_rel_l2_by_hand():
    # d = got - ref = [0, 0, -2]; |ref| = sqrt(1 + 4 + 25)
    m = oracle.compare(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 5.0]))
    assert m["max_abs"] == 2.0
    assert math.isclose(m["rel_l2"], 2.0 / math.sqrt(30.0), rel_tol=1e-15)
    assert m["nonfinite"] == 0


def test_max_is_the_largest_not_the_mean():
    # d = [0.1, -0.4, 0.2]: max |d| = 0.4, |d| = sqrt(0.21), |ref| = sqrt(3)
    m = oracle.compare(np.array([1.1, 0.6, 1.2]), np.array([1.0, 1.0, 1.0]))
    assert math.isclose(m["max_abs"], 0.4, rel_tol=1e-12)
    assert math.isclose(m["rel_l2"], math.sqrt(0.01 + 0.16 + 0.04) / math.sqrt(3.0), rel_tol=1e-12)


def test_normalised_by_the_reference_norm():
    # |d| = 1 and |ref| = 1, but |got| = 2: the figure must be 1, not 0.5
    m = oracle.compare(np.array([2.0, 0.0]), np.array([1.0, 0.0]))
    assert m["rel_l2"] == 1.0


def test_nan_in_reference_is_masked_out():
    # entries the oracle did not compute (NaN in ref) are not compared:
    # d = [0, 1] over the two finite entries, |ref| = sqrt(1 + 9)
    m = oracle.compare(np.array([1.0, 100.0, 4.0]), np.array([1.0, np.nan, 3.0]))
    assert m["max_abs"] == 1.0
    assert math.isclose(m["rel_l2"], 1.0 / math.sqrt(10.0), rel_tol=1e-15)
    assert m["nonfinite"] == 0


def test_mask_follows_the_reference_not_the_output():
    # the output's value where ref is NaN does not matter, even if it is NaN
    m = oracle.compare(np.array([np.nan, 1.0]), np.array([np.nan, 1.0]))
    assert m == {"max_abs": 0.0, "rel_l2": 0.0, "nonfinite": 0}
    m = oracle.compare(np.array([5.0, 1.0]), np.array([np.nan, 1.0]))
    assert m == {"max_abs": 0.0, "rel_l2": 0.0, "nonfinite": 0}


def test_nonfinite_output_is_counted_and_fails_every_bar():
    for bad in (np.nan, np.inf, -np.inf):
        m = oracle.compare(np.array([bad, 2.0, 3.0]), np.array([1.0, 2.0, 3.0]))
        assert m["nonfinite"] == 1
        # neither figure can pass a bar when an output is not finite
        assert not (m["max_abs"] <= 1e30) and not (m["rel_l2"] <= 1e30)
    m = oracle.compare(np.array([np.nan, np.inf]), np.array([1.0, 2.0]))
    assert m["nonfinite"] == 2


def test_zero_reference_norm_falls_back_to_absolute_l2():
    # |ref| = 0: rel_l2 is the absolute norm of the difference, sqrt(0.25 + 1)
    m = oracle.compare(np.array([0.5, -1.0]), np.array([0.0, 0.0]))
    assert m["max_abs"] == 1.0
    assert math.isclose(m["rel_l2"], math.sqrt(1.25), rel_tol=1e-15)
    m = oracle.compare(np.zeros(3), np.zeros(3))
    assert m == {"max_abs": 0.0, "rel_l2": 0.0, "nonfinite": 0}


def test_empty_comparison():
    # nothing finite to compare (all ref entries NaN): no error, zero figures
    m = oracle.compare(np.array([1.0, 2.0]), np.array([np.nan, np.nan]))
    assert m == {"max_abs": 0.0, "rel_l2": 0.0, "nonfinite": 0}


def test_shapes_and_dtypes_are_flattened_alike():
    # any shape, any float input dtype: compared element by element in fp64
    got = np.array([[1.0, 2.0], [3.0, 4.5]], dtype=np.float32)
    ref = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float64)
    m = oracle.compare(got, ref)
    assert m["max_abs"] == 0.5
    assert math.isclose(m["rel_l2"], 0.5 / math.sqrt(1 + 4 + 9 + 16), rel_tol=1e-15)

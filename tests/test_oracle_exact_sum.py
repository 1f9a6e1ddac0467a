"""Pins of the oracle's exactly rounded fp64 sum (q8ref_exact_sum), the sum
that defines the norm's sum of squares and the router's softmax denominator.

It is checked against two independent exact summations: Python's math.fsum
(Shewchuk's partials, correctly rounded) and fractions.Fraction arithmetic
converted with float(), which rounds to nearest with ties to even.  Hand
cases cover exact ties, the sticky bit below a tie, subnormal terms and
overflow.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _exact(v):
    return float(sum((Fraction(x) for x in v), Fraction(0)))


@pytest.mark.parametrize("seed", range(8))
def test_random_wide_range_against_fsum_and_fractions(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    # magnitudes spread over 2^-1074 .. 2^900, so terms overlap in every way
    mant = rng.random(n)
    expo = rng.integers(-1074, 900, n)
    v = np.ldexp(mant, expo)
    got = oracle.exact_sum(v)
    assert got == math.fsum(v.tolist())
    assert got == _exact(v.tolist())


@pytest.mark.parametrize("seed", range(4))
def test_squares_of_fp32_values(seed):
    """The norm's use: squares of fp32 values (exact in fp64), many of them."""
    rng = np.random.default_rng(100 + seed)
    h = rng.standard_normal(16384).astype(np.float32)
    h[rng.integers(0, h.size, 50)] *= np.float32(20.0)
    sq = h.astype(np.float64) ** 2
    assert oracle.exact_sum(sq) == math.fsum(sq.tolist()) == _exact(sq.tolist())


def test_order_does_not_matter():
    rng = random.Random(7)
    v = [rng.random() * 2.0 ** rng.randint(-60, 60) for _ in range(1000)]
    ref = oracle.exact_sum(v)
    for _ in range(5):
        rng.shuffle(v)
        assert oracle.exact_sum(v) == ref


# (terms, exactly rounded sum), worked by hand
HAND = [
    ([], 0.0),
    ([0.0, 0.0], 0.0),
    ([1.0, 2.0 ** -53], 1.0),                                  # exact tie, even neighbour is 1
    ([1.0 + 2.0 ** -52, 2.0 ** -53], 1.0 + 2.0 ** -51),        # exact tie, odd lower neighbour: round up
    ([1.0, 2.0 ** -53, 2.0 ** -1074], 1.0 + 2.0 ** -52),       # sticky bit far below breaks the tie
    ([1.0, 2.0 ** -54], 1.0),                                  # below half an ulp
    ([2.0 ** -1074] * 3, 3 * 2.0 ** -1074),                    # subnormal terms, exact
    ([2.0 ** -1022 - 2.0 ** -1074, 2.0 ** -1074], 2.0 ** -1022),  # subnormal carries into the normal range
    ([2.0 ** 52, 0.5], 2.0 ** 52),                             # tie at the 2^52 boundary: even
    ([2.0 ** 52 + 1, 0.5], 2.0 ** 52 + 2),                     # tie, odd: up
    ([3.0, 5.0, 7.0], 15.0),
]


@pytest.mark.parametrize("terms,want", HAND)
def test_hand_worked(terms, want):
    assert oracle.exact_sum(terms) == want
    assert _exact(terms) == want  # the worked value itself, by exact arithmetic


def test_overflow_and_invalid_terms():
    assert oracle.exact_sum([1.7e308, 1.7e308]) == math.inf
    assert math.isnan(oracle.exact_sum([1.0, -1.0]))
    assert math.isnan(oracle.exact_sum([1.0, math.inf]))
    assert math.isnan(oracle.exact_sum([math.nan]))

"""CPU check of the rule the decode kernel uses to place its slices: for
integers 0 <= n < 2^53 and 0 < d < 2^31, floor of the correctly rounded
double quotient n / d equals the integer quotient.  (When n / d is not an
integer it lies at least 1/d below the next integer, and the rounding error
is at most (n / d) 2^-53 < 1/d.)  Python floats are IEEE doubles with
correctly rounded division, the same arithmetic as the kernel's, so the
slice bounds below are the kernel's formulas on the largest operands the
host lets through: nw <= 2^20 wavefronts and a unit list shorter than 2^31.
"""
import math

import numpy as np

MAX_WAVES = 1 << 20
MAX_TOTAL = (1 << 31) - 1


def slice_start(s, total, nw):
    return math.floor((float(s) * total) / nw)


def slice_of(u, total, nw):
    return math.floor((float(u + 1) * nw - 1.0) / total)


def test_random_operands_match_integer_division():
    rng = np.random.default_rng(5)
    for _ in range(20000):
        nw = int(rng.integers(1, MAX_WAVES + 1))
        total = int(rng.integers(1, MAX_TOTAL + 1))
        s = int(rng.integers(0, nw + 1))
        u = int(rng.integers(0, total))
        assert slice_start(s, total, nw) == s * total // nw
        assert slice_of(u, total, nw) == ((u + 1) * nw - 1) // total


def test_quotients_just_below_an_integer():
    # n = k d - 1 puts the exact quotient 1/d below k: the case rounding
    # could push up to k if the bound did not hold.
    for d in (MAX_WAVES, MAX_WAVES - 1, 895, 3, MAX_TOTAL, MAX_TOTAL - 2, 12345677):
        for k in (1, 2, 1000, (1 << 52) // d, ((1 << 53) - 1) // d):
            n = k * d - 1
            if n < 0 or n >= 1 << 53:
                continue
            assert math.floor(float(n) / d) == n // d == k - 1


def test_slice_bounds_partition_the_list():
    # every entry falls in exactly one slice, and slice_of inverts slice_start
    rng = np.random.default_rng(6)
    for total, nw in [(MAX_TOTAL, MAX_WAVES), (MAX_TOTAL, 895), (4475, 895), (7, 7), (1, 1)]:
        starts = [slice_start(s, total, nw) for s in range(0, nw + 1, max(1, nw // 4096))]
        assert starts == sorted(starts) and starts[0] == 0
        assert slice_start(nw, total, nw) == total
        for u in rng.integers(0, total, 2000):
            s = slice_of(int(u), total, nw)
            assert slice_start(s, total, nw) <= u < slice_start(s + 1, total, nw)


def test_the_bound_is_needed():
    # past 2^53 a double no longer holds every integer and the rule fails
    n = (1 << 53) + 1
    assert math.floor(float(n) / 1) == n - 1 != n // 1

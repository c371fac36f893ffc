"""Pins for the grader that grades every device Top-p / Top-K selection
(``oracle/compare.py``).

The rule it grades against: papernotes.org, AdaSpark, key design 2 (S_i =
Top-p(P_i, p): the fewest preceding cubes, most probable first, whose
probabilities reach p), ties to the lower cube index, and the precision
contract's single exemption (rows whose cumulative probability lies within
1e-5 of p).  Each case below is built by hand so that one plausible grader
mistake (accepting a non-minimal set, a set that skips a more probable cube,
a swap outside the float32 window, a tie taken at the higher index) fails it.
"""
import math

import numpy as np
import pytest

from oracle import adas_oracle as O
from oracle.compare import (TOL_MASS, grade_row, grade_row_topk, grade_rows,
                            logit_error_bound)


def _softmax(z):
    e = np.exp(np.asarray(z, float) - np.max(z))
    return e / e.sum()


def test_exact_set_is_exact():
    P = np.array([0.5, 0.3, 0.2])
    assert grade_row(P, 0.7, [0, 1]) == "exact"
    assert grade_row(P, 1.0, [0, 1, 2]) == "exact"
    assert grade_row_topk(P, 2, [0, 1]) == "exact"


def test_near_threshold_alternative():
    # the oracle's sum reaches p = 0.9 at the third cube by 2e-6: a float32
    # device may fall short there and take the fourth cube as well
    P = np.array([0.4, 0.3, 0.2 + 2e-6, 0.1 - 2e-6])
    assert O.top_p(P, 0.9).tolist() == [0, 1, 2]
    assert grade_row(P, 0.9, [0, 1, 2, 3]) == "near_threshold"
    # the same alternative 1e-4 away from p is a failure (not minimal)
    P2 = np.array([0.4, 0.3, 0.2 + 1e-4, 0.1 - 1e-4])
    assert grade_row(P2, 0.9, [0, 1, 2, 3]) == "fail"
    # and stopping one cube early when the oracle sum just before the cut is
    # within 1e-5 of p (from below)
    P3 = np.array([0.4, 0.3 - 3e-6, 0.2, 0.1 + 3e-6])
    assert O.top_p(P3, 0.7).tolist() == [0, 1, 2]
    assert grade_row(P3, 0.7, [0, 1]) == "near_threshold"


def test_non_minimal_set_fails():
    P = np.array([0.5, 0.3, 0.2])
    assert grade_row(P, 0.7, [0, 1, 2]) == "fail"


def test_short_set_fails():
    P = np.array([0.5, 0.3, 0.2])
    assert grade_row(P, 0.7, [0]) == "fail"


def test_skipping_a_more_probable_cube_fails():
    # {0, 2} reaches 0.65 and is minimal, but leaves out cube 1 (P 0.3 > 0.2)
    z = np.log([0.5, 0.3, 0.2])
    P = _softmax(z)
    b = np.full(3, 1e-4)
    assert grade_row(P, 0.65, [0, 2], z, b) == "fail"


def test_swap_inside_window_is_near_tie_outside_fails():
    z = np.array([1.0, 0.5, 0.5 - 1e-7, -1.0])
    P = _softmax(z)
    p = P[0] + 0.5 * P[1]
    assert O.top_p(P, p).tolist() == [0, 1]
    b = np.full(4, 1e-6)
    assert grade_row(P, p, [0, 2], z, b) == "near_tie"
    # no window given: no ordering error is excused
    assert grade_row(P, p, [0, 2]) == "fail"
    # the same swap 1e-3 apart
    z2 = np.array([1.0, 0.5, 0.5 - 1e-3, -1.0])
    P2 = _softmax(z2)
    p2 = P2[0] + 0.5 * P2[1]
    assert grade_row(P2, p2, [0, 2], z2, b) == "fail"
    # a window that does cover 1e-3 would excuse it (the window decides)
    assert grade_row(P2, p2, [0, 2], z2, np.full(4, 6e-4)) == "near_tie"


def test_exact_tie_must_take_lower_index():
    z = np.array([1.0, 0.5, 0.5, -1.0])
    P = _softmax(z)
    assert P[1] == P[2]
    p = P[0] + 0.5 * P[1]
    assert O.top_p(P, p).tolist() == [0, 1]
    wide = np.full(4, 1.0)   # even a huge window does not excuse a tie
    assert grade_row(P, p, [0, 1], z, wide) == "exact"
    assert grade_row(P, p, [0, 2], z, wide) == "fail"
    assert grade_row_topk(P, 2, [0, 2], z, wide) == "fail"
    assert grade_row_topk(P, 2, [0, 1], z, wide) == "exact"


def test_uniform_row_takes_lowest_indices():
    n, p = 10, 0.65
    P = np.full(n, 1.0 / n)
    want = list(range(math.ceil(p * n)))
    assert O.top_p(P, p).tolist() == want
    assert grade_row(P, p, want) == "exact"
    assert grade_row(P, p, list(range(1, 8))) == "fail"
    assert grade_row(P, p, [0, 1, 2, 3, 4, 5, 7]) == "fail"


def test_malformed_sets_fail():
    P = np.array([0.5, 0.3, 0.2])
    assert grade_row(P, 0.7, []) == "fail"
    assert grade_row(P, 0.7, [1, 0]) == "fail"          # not ascending
    assert grade_row(P, 0.7, [0, 0, 1]) == "fail"       # duplicate
    assert grade_row(P, 0.7, [0, 3]) == "fail"          # out of range
    assert grade_row(P, 0.7, [-1, 0, 1]) == "fail"
    assert grade_row_topk(P, 2, [0, 1, 2]) == "fail"    # wrong size
    assert grade_row_topk(P, 2, [0, 5]) == "fail"


def test_topk_swap_window():
    z = np.array([2.0, 1.0, 1.0 - 1e-7, 0.0])
    P = _softmax(z)
    b = np.full(4, 1e-6)
    assert grade_row_topk(P, 2, [0, 2], z, b) == "near_tie"
    z2 = np.array([2.0, 1.0, 0.99, 0.0])
    assert grade_row_topk(_softmax(z2), 2, [0, 2], z2, b) == "fail"


def test_grade_rows_counts():
    P = np.array([0.5, 0.3, 0.2])
    c = grade_rows([(P, [0, 1]), (P, [0, 1, 2]), (P, [0, 1])], 0.7)
    assert c == {"exact": 2, "near_threshold": 0, "near_tie": 0, "fail": 1}


def _split3(x32):
    """A float32 value as three bf16 parts hi + mid + lo (round to nearest)."""
    def rne(v):
        u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
        return u.astype(np.uint32).view(np.float32)
    hi = rne(x32)
    r1 = (x32 - hi).astype(np.float32)
    mid = rne(r1)
    lo = rne((r1 - mid).astype(np.float32))
    return hi, mid, lo


@pytest.mark.parametrize("d", [64, 128])
def test_error_bound_covers_float32_dot_products(d):
    """The bound is a claim about float32 arithmetic: check it against float32
    computations of the logits in several summation orders (sequential,
    reversed, pairwise, and the three-way bf16 split of the mean key), on
    inputs shaped like the workloads and on adversarial ones with large
    cancellation."""
    rng = np.random.default_rng(d)
    for trial in range(40):
        q = rng.standard_normal(d).astype(np.float32)
        q = q.view(np.uint32)
        q = ((q + 0x7FFF + ((q >> 16) & 1)) >> 16 << 16).view(np.float32)   # bf16 values
        kb = (rng.standard_normal((50, d)) * (1.5 if trial % 2 else 1.0)).astype(np.float64)
        if trial % 5 == 0:   # cancellation: mean keys nearly orthogonal to q
            qd = q.astype(np.float64)
            kb -= np.outer(kb @ qd / (qd @ qd), qd) * 0.999
        z = O.selection_logits(q.astype(np.float64), kb)
        bound = logit_error_bound(q.astype(np.float64), kb, z)
        kb32 = kb.astype(np.float32)
        sc = np.float32(1.0 / math.sqrt(d))
        prods = (q[None, :] * kb32)                              # float32 products
        variants = []
        acc = np.zeros(50, np.float32)
        for i in range(d):
            acc = (acc + prods[:, i]).astype(np.float32)
        variants.append(acc)
        acc = np.zeros(50, np.float32)
        for i in reversed(range(d)):
            acc = (acc + prods[:, i]).astype(np.float32)
        variants.append(acc)
        variants.append(np.sum(prods, axis=1, dtype=np.float32))
        hi, mid, lo = _split3(kb32)
        parts = np.concatenate([q[None, :] * hi, q[None, :] * mid, q[None, :] * lo], axis=1)
        acc = np.zeros(50, np.float32)
        for i in range(parts.shape[1]):
            acc = (acc + parts[:, i]).astype(np.float32)
        variants.append(acc)
        for v in variants:
            z32 = (v * sc).astype(np.float32).astype(np.float64)
            assert np.all(np.abs(z32 - z) <= bound)
    # and it is not vacuous: far below the logit spacing of a typical row
    assert np.median(bound) < 1e-2

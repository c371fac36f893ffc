"""Pins for the oracle's selection softmax (O3/O4) and Top-p sets (O5).

AdaSpark, papernotes.org, key design 2: P_i = Softmax over the preceding
cubes of q . kbar_j / sqrt(d_k); S_i = Top-p(P_i, p); key design 4: one
threshold p.  The listing's Figure 2 caption: each query selects among
*preceding* cubes.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import adas_oracle as O
from tests.conftest import GOLDEN


def test_topp_golden():
    gold = json.load(open(os.path.join(GOLDEN, "topp_cases.json")))
    for case in gold["cases"]:
        got = O.top_p(np.array(case["P"], dtype=np.float64), case["p"]).tolist()
        assert got == case["S"], case


def test_softmax_golden():
    gold = json.load(open(os.path.join(GOLDEN, "softmax_cases.json")))
    for case in gold["cases"]:
        P = O.selection_probabilities(np.array(case["q"]), np.array(case["kbar"]))
        np.testing.assert_allclose(P, case["P"], rtol=0, atol=1e-15)


def _random_P(rng, n, temp):
    return O.softmax(rng.standard_normal(n) * temp)


def test_softmax_rows_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(0)
    for n in (1, 2, 7, 100, 1023):
        z = rng.standard_normal((5, n)) * 3
        P = O.softmax(z)
        assert np.all(np.abs(P.sum(axis=1) - 1) <= 1e-12)
        np.testing.assert_allclose(O.softmax(z + 123.25), P, rtol=1e-12, atol=1e-15)
    assert O.softmax(np.array([[4.2]])).tolist() == [[1.0]]
    assert O.softmax(np.zeros((3, 0))).shape == (3, 0)


def test_logit_scale_is_inverse_sqrt_dk():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(64)
    kb = rng.standard_normal((10, 64))
    z = O.selection_logits(q, kb)
    np.testing.assert_allclose(z, [np.dot(q, kb[j]) / 8.0 for j in range(10)], rtol=1e-13)


@pytest.mark.parametrize("p", [0.05, 0.3, 0.5, 0.7, 0.9, 0.99])
def test_topp_reaches_p_and_is_minimal(p):
    rng = np.random.default_rng(int(p * 1000))
    for n in (1, 2, 3, 10, 64, 500):
        for temp in (0.1, 1.0, 3.0):
            P = _random_P(rng, n, temp)
            S = O.top_p(P, p)
            assert np.all(np.diff(S) > 0), "ascending, no duplicates"
            mass = P[S].sum()
            assert mass >= p - 1e-12 or len(S) == n
            assert mass - P[S].min() < p, "dropping the smallest member must fall short of p"
            # every unselected cube has P no larger than every selected one
            rest = np.setdiff1d(np.arange(n), S)
            if len(rest):
                assert P[rest].max() <= P[S].min()


def _brute_force_topp(P, p):
    """Smallest cardinality k for which some k-subset reaches p, and the best
    mass among k-subsets, by enumerating every subset."""
    n = len(P)
    for k in range(1, n + 1):
        best = max(sum(P[list(s)]) for s in itertools.combinations(range(n), k))
        if best >= p:
            return k, best
    return n, sum(P)


def test_topp_matches_subset_enumeration():
    rng = np.random.default_rng(2)
    for trial in range(150):
        n = int(rng.integers(1, 13))
        P = _random_P(rng, n, float(rng.choice([0.3, 1.0, 2.5])))
        p = float(rng.uniform(0.05, 0.98))
        S = O.top_p(P, p)
        k, best = _brute_force_topp(P, p)
        assert len(S) == k, (P, p)
        assert abs(P[S].sum() - best) < 1e-12, "the nucleus is a max-mass set of its size"


def test_topp_uniform_takes_lowest_indices():
    for n, p in [(10, 0.65), (10, 0.05), (7, 0.5), (33, 0.71), (1023, 0.7), (4096, 0.3)]:
        P = np.full(n, 1.0 / n)
        S = O.top_p(P, p)
        assert S.tolist() == list(range(math.ceil(p * n)))


def test_topp_limits():
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(1, 200))
        P = _random_P(rng, n, 2.0)
        assert O.top_p(P, 1e-9).tolist() == [int(np.argmax(P))]
        assert O.top_p(P, 1.0).tolist() == list(range(n))
    P = np.array([0.2, 0.4, 0.4])
    assert O.top_p(P, 1e-9).tolist() == [1], "argmax ties go to the lower index"


def test_topp_batch_equals_scalar():
    rng = np.random.default_rng(4)
    for n in (1, 5, 64, 300):
        P = O.softmax(rng.standard_normal((40, n)) * 2)
        P[3] = 1.0 / n                                    # a uniform row (ties)
        P[4, : n // 2] = P[4, n // 2: 2 * (n // 2)] if n > 1 else P[4, :0]
        P[4] /= P[4].sum()
        for p in (0.3, 0.7, 0.9, 1.0):
            counts, mask = O.top_p_batch(P, p)
            for r in range(P.shape[0]):
                S = O.top_p(P[r], p)
                assert counts[r] == len(S)
                assert np.nonzero(mask[r])[0].tolist() == S.tolist()


def test_entropy_adaptivity():
    """Key design 2: spread-out (high-entropy) P selects more cubes than a
    peaked one at the same p."""
    rng = np.random.default_rng(5)
    z = rng.standard_normal(200)
    sizes = [len(O.top_p(O.softmax(z * t), 0.7)) for t in (0.1, 0.5, 1.0, 2.0, 5.0)]
    assert sizes == sorted(sizes, reverse=True) and sizes[0] > sizes[-1]


def test_video_row_candidates_are_preceding_cubes():
    wl = workloads.get("tiny")
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, _ = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    kbar = O.mean_keys(k_cube, g)
    sel = O.select_video_rows(q_cube, kbar, g, wl.p)
    assert len(sel) == g.N
    for (hq, pos), S in sel.items():
        c = pos // g.S
        if c == 0:
            assert len(S) == 0, "the first cube has no candidates"
        else:
            assert 1 <= len(S) <= c and S.max() < c
        if c == 1:
            assert S.tolist() == [0]


def test_identical_cubes_give_uniform_selection():
    """All cubes share one mean key -> P uniform -> lowest ceil(p * c) cubes."""
    g = O.Geometry(4, 4, 4, 1, 2, 2)                    # 16 cubes of 4
    rng = np.random.default_rng(6)
    key = rng.standard_normal(8).astype(np.float32)
    k_cube = np.broadcast_to(key, (1, g.N, 8)).copy()
    q_cube = rng.standard_normal((2, g.N, 8)).astype(np.float32)
    kbar = O.mean_keys(k_cube, g)
    p = 0.65
    sel = O.select_video_rows(q_cube, kbar, g, p)
    for (hq, pos), S in sel.items():
        c = pos // g.S
        assert S.tolist() == list(range(math.ceil(p * c) if c else 0))


def test_extra_rows_select_over_all_cubes():
    wl = workloads.get("tiny").replace(n_decode=5, video_queries=False)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    k_cube, _ = O.partition(data["k"], g)
    kbar = O.mean_keys(k_cube, g)
    sel = O.select_extra_rows(data["q_text"], kbar, 0.9)
    for (hq, m), S in sel.items():
        P = O.selection_probabilities(O.to_f64(data["q_text"][m, hq]), kbar[0])
        assert len(P) == g.n_cubes
        assert S.tolist() == O.top_p(P, 0.9).tolist()


# --- Top-K, the fixed-budget strategy of the listing's Table 4 -----------------------
def _brute_force_topk(P, k):
    """All k-subsets; the answer is the one of largest mass, ties broken by the
    lexicographically smallest sorted index tuple."""
    n = len(P)
    if k >= n:
        return list(range(n))
    best = None
    for sub in itertools.combinations(range(n), k):
        key = (-sum(P[list(sub)]), sub)
        best = key if best is None or key < best else best
    return list(best[1])


def test_topk_matches_subset_enumeration():
    rng = np.random.default_rng(11)
    for trial in range(120):
        n = int(rng.integers(1, 11))
        P = _random_P(rng, n, float(rng.choice([0.3, 1.0, 2.5])))
        if trial % 3 == 0:
            P = np.round(P * 4) / 4 + 1e-3   # coarse values: many exact ties
            P /= P.sum()
        k = int(rng.integers(1, n + 2))
        assert O.top_k(P, k).tolist() == _brute_force_topk(P, k), (P, k)


def test_topk_limits_and_ties():
    P = np.array([0.1, 0.3, 0.2, 0.3, 0.1])
    assert O.top_k(P, 1).tolist() == [1], "equal P: the lower index first"
    assert O.top_k(P, 2).tolist() == [1, 3]
    assert O.top_k(P, 4).tolist() == [0, 1, 2, 3]
    assert O.top_k(P, 9).tolist() == [0, 1, 2, 3, 4], "fewer candidates than k: all"
    assert O.top_k(np.zeros(0), 3).tolist() == []
    n = 37
    assert O.top_k(np.full(n, 1.0 / n), 10).tolist() == list(range(10)), "uniform: lowest indices"
    with pytest.raises(ValueError):
        O.top_k(P, 0)


def test_topk_is_nested_and_agrees_with_topp_at_its_own_mass():
    rng = np.random.default_rng(12)
    for _ in range(60):
        n = int(rng.integers(2, 300))
        P = _random_P(rng, n, 2.0)
        prev = set()
        for k in range(1, min(n, 40)):
            S = set(O.top_k(P, k).tolist())
            assert prev < S and len(S) == k, "sets grow by one cube per unit of k"
            prev = S
        # with distinct P, Top-k is the Top-p set at p = mass of the k largest
        k = int(rng.integers(1, n))
        srt = np.sort(P)[::-1]
        if srt[k - 1] > srt[k]:
            p = float(np.sum(srt[:k]))
            assert O.top_p(P, p * (1 - 1e-12)).tolist() == O.top_k(P, k).tolist()


def test_topk_rows_select_preceding_cubes_only():
    wl = workloads.get("tiny").replace(name="tiny_topk")
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, _ = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    kbar = O.mean_keys(k_cube, g)
    sel = O.select_video_rows(q_cube, kbar, g, p=0.7, k=3)
    for (hq, pos), S in sel.items():
        c = pos // g.S
        assert len(S) == min(3, c) and all(0 <= j < c for j in S)
        P = O.selection_probabilities(O.to_f64(q_cube[hq, pos][None]), kbar[0, :c])[0]
        assert S.tolist() == O.top_k(P, 3).tolist()

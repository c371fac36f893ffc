"""Grading a device selection against the oracle -- test infrastructure only.

Top-p sets are decided by floating-point sums, so a device that computes the
selection softmax in float32 can legitimately differ from the float64 oracle
on rows whose cumulative probability sits next to p, or whose cut falls
between two cubes of (numerically) equal probability.  Each row gets one
grade:

* ``exact``          -- same set;
* ``near_threshold`` -- different set, and the oracle's cumulative sum just
  before or at its cut lies within ``tol_mass`` of p;
* ``near_tie``       -- same size, different members, and every swapped cube's
  probability is within ``tol_rel`` (relative) of the cut probability;
* ``fail``           -- anything else, or a device set that is not a valid
  Top-p set for P perturbed within those tolerances.
"""
from __future__ import annotations

import numpy as np

from .adas_oracle import top_k, top_p

TOL_MASS = 1e-5
TOL_REL = 1e-5


def grade_row(P: np.ndarray, p: float, S_dev, tol_mass: float = TOL_MASS,
              tol_rel: float = TOL_REL) -> str:
    S_dev = np.asarray(S_dev, dtype=np.int64)
    S_ref = top_p(P, p)
    if S_dev.shape == S_ref.shape and np.array_equal(S_dev, S_ref):
        return "exact"
    n = len(P)
    if len(S_dev) == 0 or len(np.unique(S_dev)) != len(S_dev) or np.any(np.diff(S_dev) <= 0):
        return "fail"
    if S_dev.min() < 0 or S_dev.max() >= n:
        return "fail"
    # validity of the device set under small perturbations of P and p
    mass = float(P[S_dev].sum())
    if mass < p - tol_mass:
        return "fail"
    if mass - float(P[S_dev].min()) >= p + tol_mass:
        return "fail"
    rest = np.setdiff1d(np.arange(n), S_dev)
    if len(rest) and float(P[S_dev].min()) < float(P[rest].max()) * (1 - tol_rel):
        return "fail"
    # classify
    order = np.lexsort((np.arange(n), -P))
    cum = np.cumsum(P[order])
    k = len(S_ref)
    s_k = cum[k - 1]
    s_km1 = cum[k - 2] if k >= 2 else 0.0
    if abs(s_k - p) <= tol_mass or abs(s_km1 - p) <= tol_mass:
        return "near_threshold"
    if len(S_dev) == k:
        cut = P[order[k - 1]]
        diff = np.setxor1d(S_dev, S_ref)
        if np.all(np.abs(P[diff] - cut) <= tol_rel * cut):
            return "near_tie"
    return "fail"


def grade_rows(items, p: float):
    """items: iterable of (P, S_dev); returns a dict of grade counts."""
    counts = {"exact": 0, "near_threshold": 0, "near_tie": 0, "fail": 0}
    for P, S in items:
        counts[grade_row(P, p, S)] += 1
    return counts


def grade_row_topk(P: np.ndarray, k: int, S_dev, tol_rel: float = TOL_REL) -> str:
    """Top-K counterpart: ``exact``; ``near_tie`` when the device set has the
    right size and differs only by cubes whose probability is within
    ``tol_rel`` (relative) of the oracle's k-th largest; ``fail`` otherwise."""
    S_dev = np.asarray(S_dev, dtype=np.int64)
    S_ref = top_k(P, k)
    if S_dev.shape == S_ref.shape and np.array_equal(S_dev, S_ref):
        return "exact"
    n = len(P)
    if len(S_dev) != len(S_ref) or len(S_dev) == 0:
        return "fail"
    if np.any(np.diff(S_dev) <= 0) or S_dev.min() < 0 or S_dev.max() >= n:
        return "fail"
    cut = P[S_ref].min()
    diff = np.setxor1d(S_dev, S_ref)
    if np.all(np.abs(P[diff] - cut) <= tol_rel * cut):
        return "near_tie"
    return "fail"

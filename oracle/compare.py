"""Grading a device selection against the oracle -- test infrastructure only.

Top-p sets are decided by floating-point sums (papernotes.org, AdaSpark, key
design 2: S_i = Top-p(P_i, p), the smallest set of preceding cubes whose
probabilities reach p; ties to the lower cube index).  A device that scores
and sums in float32 can legitimately differ from the float64 oracle in two
ways, and only in these:

* the row's cumulative probability sits next to p: the oracle's sum just
  before or at its cut lies within ``tol_mass`` (1e-5) of p.  This is the one
  exemption the method's precision contract names; the row is graded
  ``near_threshold`` and counted;
* two cubes straddle the cut with logits closer than the float32 scoring
  error can resolve: the device may order them the other way.  The window is
  not a guess: ``logit_error_bound`` gives, per candidate, a worst-case bound
  on |z_device - z| for a float32 dot product of d terms (derivation in its
  docstring).  A same-size set whose every swapped pair lies inside the sum
  of the two candidates' bounds is graded ``near_tie`` and counted.

Exact ties are never excused: two cubes whose float64 probabilities are equal
have bit-identical mean keys, so the device computes bit-identical logits for
them too and must take the lower index, as the oracle does.

Each row gets one grade: ``exact``, ``near_threshold``, ``near_tie`` or
``fail``.  Every non-exact grade also requires the device set to be a valid
Top-p set under those tolerances (strictly ascending ids in range, reaches
p - tol_mass, minimal up to tol_mass, and no unselected cube above a selected
one beyond the error window).
"""
from __future__ import annotations

import math

import numpy as np

from .adas_oracle import top_k, top_p

TOL_MASS = 1e-5
U32 = 2.0 ** -23      # float32 relative rounding bound with directed rounding (twice RNE's)


def logit_error_bound(q: np.ndarray, kbar: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Worst-case |z_device - z| per candidate, for z = q . kbar_j / sqrt(d).

    q: [d] float64 (the exact bf16 or float32 query), kbar: [n, d] float64
    (the exact mean keys), z: [n] the float64 logits.  Terms, each a standard
    first-order bound (Higham, Accuracy and Stability of Numerical Algorithms,
    section 3.1: a sum of m terms in floating point is within (m-1)u times
    the sum of their magnitudes, whatever the order):

    * the mean keys are stored as float32: |kbar_f32 - kbar| <= u |kbar|
      elementwise, i.e. u * sum_i |q_i kbar_ij| on the dot product;
    * the dot product itself: at most 3d products (a float32 mean key split
      into three bf16 parts for the bf16 matrix product; d float32 fused
      multiply-adds otherwise), each exact or rounded once, then summed:
      (3d + 1) u * sum_i |q_i kbar_ij|;
    * the 1/sqrt(d) scale is a rounded float32 constant and the product is
      rounded: 3u |z_j|;
    * the exponent of the softmax takes z_j - max z rounded and scaled by a
      rounded log2(e): 3u (|z_j| + |max z|), plus a few ulps of exp2 on
      outputs near 1: 4u.

    u is taken as 2^-23, which also covers rounding toward zero.  The bound
    is worst case: the observed error is orders of magnitude smaller."""
    d = q.shape[-1]
    s = np.abs(kbar) @ np.abs(q)
    zmax = float(np.abs(z).max()) if len(z) else 0.0
    return (3 * d + 2) * U32 * s / math.sqrt(d) + 3 * U32 * np.abs(z) + 3 * U32 * (np.abs(z) + zmax) + 4 * U32


def _basic_checks(S_dev: np.ndarray, n: int) -> bool:
    if len(S_dev) and (S_dev.min() < 0 or S_dev.max() >= n):
        return False
    return bool(np.all(np.diff(S_dev) > 0))


def _window_ok(z, bound, a, b) -> bool:
    """Can the device, within its error bounds, rank cube a at or above cube b
    although the float64 logits say z_a < z_b?"""
    return z[b] - z[a] <= bound[a] + bound[b]


def _order_ok(z, bound, chosen, rest) -> bool:
    """No unselected cube b outranks a selected cube a beyond their error
    window: for every pair with z_a < z_b, z_b - z_a <= bound_a + bound_b."""
    o = np.argsort(z[chosen], kind="stable")
    zs = z[chosen][o]
    low = np.minimum.accumulate((z[chosen] + bound[chosen])[o])   # min of z_a + bound_a over a prefix
    cnt = np.searchsorted(zs, z[rest], side="left")                # selected cubes strictly below each b
    has = cnt > 0
    if not np.any(has):
        return True
    return bool(np.all(z[rest][has] - bound[rest][has] <= low[cnt[has] - 1]))


def _tie_rule_ok(P, S_dev, sel) -> bool:
    """Exactly equal probabilities: a selected cube must never have an
    unselected equal-probability cube of lower index."""
    if len(S_dev) == 0:
        return True
    vals, inv = np.unique(P, return_inverse=True)
    for v in np.unique(inv[S_dev]):
        members = np.nonzero(inv == v)[0]
        if len(members) < 2:
            continue
        taken = sel[members]
        # taken must be a prefix of the (ascending) members
        if np.any(taken[1:] & ~taken[:-1]):
            return False
    return True


def grade_row(P: np.ndarray, p: float, S_dev, z=None, bound=None,
              tol_mass: float = TOL_MASS) -> str:
    """Grade one device Top-p set.  P: float64 probabilities of the row's
    candidates; z, bound: float64 logits and ``logit_error_bound`` (without
    them no ordering error is excused)."""
    S_dev = np.asarray(S_dev, dtype=np.int64)
    S_ref = top_p(P, p)
    if S_dev.shape == S_ref.shape and np.array_equal(S_dev, S_ref):
        return "exact"
    n = len(P)
    if n == 0 or len(S_dev) == 0 or not _basic_checks(S_dev, n):
        return "fail"
    if z is None:
        z = np.log(np.maximum(P, np.finfo(float).tiny))
        bound = np.zeros(n)
    sel = np.zeros(n, dtype=bool)
    sel[S_dev] = True
    if not _tie_rule_ok(P, S_dev, sel):
        return "fail"
    # validity of the device set under the tolerances
    mass = float(P[S_dev].sum())
    if mass < p - tol_mass:
        return "fail"
    if p < 1.0 and mass - float(P[S_dev].min()) >= p + tol_mass:
        return "fail"
    if not sel.all() and not _order_ok(z, bound, S_dev, np.nonzero(~sel)[0]):
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
        extra = np.setdiff1d(S_dev, S_ref)      # device took these instead of ...
        missing = np.setdiff1d(S_ref, S_dev)    # ... these
        if all(_window_ok(z, bound, a, b) for a in extra for b in missing):
            return "near_tie"
    return "fail"


def grade_rows(items, p: float):
    """items: iterable of (P, S_dev) or (P, S_dev, z, bound); returns grade counts."""
    counts = {"exact": 0, "near_threshold": 0, "near_tie": 0, "fail": 0}
    for it in items:
        counts[grade_row(it[0], p, *it[1:])] += 1
    return counts


def grade_row_topk(P: np.ndarray, k: int, S_dev, z=None, bound=None) -> str:
    """Top-K counterpart (thelatestinai.com listing, Table 4, "Top-K" row):
    ``exact``; ``near_tie`` when the device set has the right size and every
    cube it took instead of an oracle cube lies inside the pair's float32
    error window (``logit_error_bound``); ``fail`` otherwise, and always when
    exactly equal probabilities were not resolved to the lower index."""
    S_dev = np.asarray(S_dev, dtype=np.int64)
    S_ref = top_k(P, k)
    if S_dev.shape == S_ref.shape and np.array_equal(S_dev, S_ref):
        return "exact"
    n = len(P)
    if len(S_dev) != len(S_ref) or len(S_dev) == 0 or not _basic_checks(S_dev, n):
        return "fail"
    if z is None:
        z = np.log(np.maximum(P, np.finfo(float).tiny))
        bound = np.zeros(n)
    sel = np.zeros(n, dtype=bool)
    sel[S_dev] = True
    if not _tie_rule_ok(P, S_dev, sel):
        return "fail"
    extra = np.setdiff1d(S_dev, S_ref)
    missing = np.setdiff1d(S_ref, S_dev)
    if all(_window_ok(z, bound, a, b) for a in extra for b in missing):
        return "near_tie"
    return "fail"

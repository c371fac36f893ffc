"""Whole-layer check of the device's Top-p (or Top-K) lists against the oracle.

Every row's set is compared, not a sample: the oracle computes each row's
Top-p set (papernotes.org, AdaSpark, key design 2: S_i = Top-p(P_i, p)) and
reduces it to (count, signature), where the signature is the sum of a fixed
random 40-bit tag per cube id over the set.  The device's lists are reduced
the same way on the GPU, so only two small arrays per head cross to the
host.  Rows whose pair differs are re-graded one by one with
``oracle.compare`` (float64 probabilities, float32 error window).  Distinct
sets share a signature with probability about 2^-40 per row.

This module imports NumPy and the oracle only (no torch), so its per-head
work runs in worker processes that never touch the GPU.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

from oracle import adas_oracle as O
from oracle.compare import TOL_MASS

TAG_BITS = 40


def tags(n_cubes: int) -> np.ndarray:
    """Fixed random tag per cube id (seeded; test bookkeeping only)."""
    return np.random.default_rng(20240607).integers(0, 1 << TAG_BITS, size=n_cubes, dtype=np.int64)


def _near_flags(P: np.ndarray, p: float, k: np.ndarray) -> np.ndarray:
    """Rows whose oracle sum at or just before the cut lies within 1e-5 of p."""
    rows, n = P.shape
    if n == 0 or p >= 1.0:
        return np.zeros(rows, bool)
    srt = -np.sort(-P, axis=1)
    cum = np.cumsum(srt, axis=1)
    r = np.arange(rows)
    s_k = cum[r, k - 1]
    s_km1 = np.where(k >= 2, cum[r, np.maximum(k - 2, 0)], 0.0)
    return (np.abs(s_k - p) <= TOL_MASS) | (np.abs(s_km1 - p) <= TOL_MASS)


def _rows_signature(P: np.ndarray, p: float, tag: np.ndarray):
    k, mask = O.top_p_batch(P, p)
    sig = (mask * tag[None, :P.shape[1]]).sum(axis=1) if P.shape[1] else np.zeros(len(P), np.int64)
    return k, sig.astype(np.int64), _near_flags(P, p, k)


def _rows_signature_topk(P: np.ndarray, k: int, tag: np.ndarray):
    """Top-K counterpart of _rows_signature: each row's set from the oracle's
    ``top_k``; no near-threshold notion (near is all False)."""
    rows, n = P.shape
    mask = np.zeros((rows, n), bool)
    for r in range(rows):
        mask[r, O.top_k(P[r], k)] = True
    sig = (mask * tag[None, :n]).sum(axis=1) if n else np.zeros(rows, np.int64)
    return mask.sum(axis=1).astype(np.int32), sig.astype(np.int64), np.zeros(rows, bool)


def video_head(q_head: np.ndarray, kbar_g: np.ndarray, S: int, p: float, k: int | None = None):
    """One query head's video rows, cube by cube: q_head [N][d] (cube
    layout, bf16 bits or float32), kbar_g [Nc][d] float64 (exact means).
    Top-K sets instead of Top-p when k is given.
    Returns (counts [N] int32, signatures [N] int64, near [N] bool)."""
    N, d = q_head.shape
    nc = N // S
    tag = tags(nc)
    counts = np.zeros(N, np.int32)
    sig = np.zeros(N, np.int64)
    near = np.zeros(N, bool)
    q64 = O.to_f64(q_head)
    for c in range(1, nc):
        P = O.selection_probabilities(q64[c * S:(c + 1) * S], kbar_g[:c])
        cnt, s, nf = _rows_signature(P, p, tag) if k is None else _rows_signature_topk(P, k, tag)
        counts[c * S:(c + 1) * S] = cnt
        sig[c * S:(c + 1) * S] = s
        near[c * S:(c + 1) * S] = nf
    return counts, sig, near


def extra_head(q_rows: np.ndarray, kbar_g: np.ndarray, p: float, k: int | None = None):
    """Extra (text / decode) rows of one head over every cube: q_rows [m][d]."""
    tag = tags(kbar_g.shape[0])
    P = O.selection_probabilities(O.to_f64(q_rows), kbar_g)
    return _rows_signature(P, p, tag) if k is None else _rows_signature_topk(P, k, tag)


def _video_task(args):
    # one BLAS thread per worker process: the pool supplies the parallelism
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return video_head(*args)


def oracle_signatures(ref, p: float, workers: int | None = None, k: int | None = None):
    """(counts, signatures, near) of every row, shaped [Hq][rows_per_head],
    video rows first (Top-K sets when k is given).  Per-head work runs in a
    pool of spawned processes."""
    wl, g = ref.wl, ref.g
    Hq = wl.n_q_heads
    R = ref.rows_per_head
    counts = np.zeros((Hq, R), np.int32)
    sig = np.zeros((Hq, R), np.int64)
    near = np.zeros((Hq, R), bool)
    nv = g.N if wl.video_queries else 0
    if wl.video_queries:
        tasks = [(ref.q_cube[hq], ref.kbar[ref.kv(hq)], g.S, p, k) for hq in range(Hq)]
        if workers is None:
            workers = min(16, len(os.sched_getaffinity(0)), Hq)
        if workers > 1:
            with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
                results = list(ex.map(_video_task, tasks))
        else:
            results = [video_head(*t) for t in tasks]
        for hq, (c, s, nf) in enumerate(results):
            counts[hq, :nv], sig[hq, :nv], near[hq, :nv] = c, s, nf
    if ref.n_extra:
        for hq in range(Hq):
            c, s, nf = extra_head(ref.data["q_text"][:, hq], ref.kbar[ref.kv(hq)], p, k)
            counts[hq, nv:], sig[hq, nv:], near[hq, nv:] = c, s, nf
    return counts, sig, near


def list_signature_numpy(sel_count, sel_idx, ref) -> np.ndarray:
    """The device-side reduction written with NumPy, for CPU tests of the
    bookkeeping: signature of every row from the packed lists."""
    g, wl = ref.g, ref.wl
    tag = tags(g.n_cubes)
    Hq, R = sel_count.shape
    sig = np.zeros((Hq, R), np.int64)
    nv = g.N if wl.video_queries else 0
    for hq in range(Hq):
        for pos in range(nv):
            off = ref.video_off(hq, pos)
            sig[hq, pos] = tag[sel_idx[off:off + sel_count[hq, pos]]].sum()
        for m in range(ref.n_extra):
            off = ref.extra_off(hq, m)
            sig[hq, nv + m] = tag[sel_idx[off:off + sel_count[hq, nv + m]]].sum()
    return sig

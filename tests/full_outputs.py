"""Whole-layer check of the device's attention outputs against the oracle.

Every row's output is recomputed by the oracle (papernotes.org, AdaSpark, key
design 2: exact attention over the selected cubes and the row's own cube;
text and decode rows: the selected cubes, plus causal text keys in a text
prefill) over the device's own selection list of that row, and compared
element by element with the device's bf16 output.

This module imports NumPy and the oracle only (no torch).  Worker processes
rebuild the layer's inputs from the workload's seed once each, so only the
row lists and the device outputs of each task cross process boundaries.
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

import workloads
from oracle import adas_oracle as O

_STATE = {}


def _init(wl):
    from threadpoolctl import threadpool_limits
    _STATE["limits"] = threadpool_limits(limits=1)  # the pool supplies the parallelism
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    _STATE["g"] = g
    _STATE["k_cube"] = O.partition(data["k"], g)[0]
    _STATE["v_cube"] = O.partition(data["v"], g)[0]
    _STATE["q_cube"] = O.partition(data["q"], g)[0] if wl.video_queries else None
    _STATE["q_text"] = data.get("q_text")
    _STATE["k_text"] = data["k_text"] if wl.text_kv else None
    _STATE["v_text"] = data["v_text"] if wl.text_kv else None


def _task(args):
    """args: (kind, hq, [(row, cubes)], device outputs [n][d] as bf16 bits).
    Returns (max-abs error, sum of abs errors, element count)."""
    kind, hq, rows, dev = args
    s = _STATE
    worst, total = 0.0, 0.0
    for (i, cubes), got in zip(rows, dev):
        if kind == "v":
            o = O.attention_video_row(s["q_cube"], s["k_cube"], s["v_cube"], s["g"], hq, i, cubes)
        else:
            o = O.attention_extra_row(s["q_text"], s["k_cube"], s["v_cube"], s["g"], hq, i, cubes,
                                      s["k_text"], s["v_text"])
        e = np.abs(O.to_f64(got) - o)
        worst = max(worst, float(e.max()))
        total += float(e.sum())
    return worst, total, len(rows) * dev.shape[-1]


def check_lists(cnt, idx, offs, n_cand):
    """Structural check of device lists: ascending ids below the row's
    candidate count, count within it.  offs, n_cand: per row."""
    for o, c, n in zip(offs, cnt, n_cand):
        lst = idx[o:o + c]
        assert 0 <= c <= n, (o, c, n)
        if c:
            assert lst[0] >= 0 and lst[-1] < n and np.all(np.diff(lst) > 0), (o, lst[:8])


def full_outputs(wl, sel_count, sel_idx, out_raster, out_extra, perm, chunk_rows=2048, workers=None,
                 positions=None):
    """Compare every row (every extra row, and the video rows at the cube
    positions ``positions`` of every head when given).  sel_count
    [Hq][rows_per_head], sel_idx (flat), out_raster [N][Hq][d] and out_extra
    [n_extra][Hq][d] as bf16 bits, perm [N] (cube position -> raster token).
    Returns (max-abs, mean-abs, rows)."""
    g = O.Geometry.of(wl)
    Hq, S, Nc = wl.n_q_heads, g.S, g.n_cubes
    n_extra = wl.n_text + wl.n_decode
    capv = S * Nc * (Nc - 1) // 2 if wl.video_queries else 0
    nv = g.N if wl.video_queries else 0
    tasks = []
    n_rows = 0
    for hq in range(Hq):
        if wl.video_queries:
            pos = np.arange(g.N) if positions is None else np.asarray(positions)
            c = pos // S
            offs = hq * capv + S * c * (c - 1) // 2 + (pos - c * S) * c
            cnt = sel_count[hq, pos]
            check_lists(cnt, sel_idx, offs, c)
            rows = [(int(p), sel_idx[o:o + k]) for p, o, k in zip(pos, offs, cnt)]
            dev = out_raster[perm[pos], hq]  # in the order of pos
            for a in range(0, len(pos), chunk_rows):
                tasks.append(("v", hq, rows[a:a + chunk_rows], dev[a:a + chunk_rows]))
            n_rows += len(pos)
        if n_extra:
            offs = Hq * capv + (hq * n_extra + np.arange(n_extra)) * Nc
            cnt = sel_count[hq, nv:]
            check_lists(cnt, sel_idx, offs, np.full(n_extra, Nc))
            rows = [(m, sel_idx[o:o + k]) for m, o, k in zip(range(n_extra), offs, cnt)]
            per = max(1, min(chunk_rows, n_extra // 2 or 1))
            for a in range(0, n_extra, per):
                tasks.append(("x", hq, rows[a:a + per], out_extra[a:a + per, hq]))
            n_rows += n_extra
    worst, mean = run_tasks(wl, tasks, workers)
    return worst, mean, n_rows


def run_tasks(wl, tasks, workers=None):
    """Run (kind, hq, [(row, cubes)], device outputs) tasks in a pool of
    spawned workers; returns (max-abs, mean-abs) over every element."""
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)), len(tasks))
    res = []
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                             initializer=_init, initargs=(wl,)) as ex:
        for r in ex.map(_task, tasks):
            res.append(r)
            if len(res) % max(1, len(tasks) // 8) == 0:
                print(f"  oracle outputs: {len(res)} of {len(tasks)} tasks done", flush=True)
    return max(r[0] for r in res), sum(r[1] for r in res) / sum(r[2] for r in res)

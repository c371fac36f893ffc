"""CPU oracle for the gradients of AdaS-Attn's sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; it never calls the
HIP library.

The pages adapt a pretrained backbone to the sparse pattern with a short
fine-tuning (papernotes.org, "损失函数 / 训练策略"), which needs the gradient of
the attention of key design 2 with respect to Q, K and V.  The Top-p sets are
discrete choices, so they are held fixed: no gradient flows into the
selection or into the mean keys.  For one row with keys k_j, values v_j over
its attended set A (selected cubes, own cube, causal text) and scale
c = 1/sqrt(d):

    s_j = c q.k_j,  p = softmax(s),  o = sum_j p_j v_j
    dv_j += p_j do                      (each key collects from every row)
    dp_j = do . v_j,  D = sum_j p_j dp_j (= do . o)
    ds_j = p_j (dp_j - D)
    dq = c sum_j ds_j k_j,  dk_j += c ds_j q

written out in float64 NumPy.  The row's log-sum-exp of s is returned too
(the forward hands it to the backward).
"""
from __future__ import annotations

import math

import numpy as np

from .adas_oracle import Geometry, _kv_head, cube_coords, to_f64

__all__ = ["attend_grad", "attention_grads", "row_weights"]


def attend_grad(q: np.ndarray, keys: np.ndarray, values: np.ndarray, do: np.ndarray):
    """One row: returns (o, lse, dq, dk [n][d], dv [n][d]) in float64."""
    c = 1.0 / math.sqrt(q.shape[-1])
    s = c * (keys @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    p = e / z
    o = p @ values
    dv = np.outer(p, do)
    dp = values @ do
    D = float(p @ dp)
    ds = p * (dp - D)
    dq = c * (ds @ keys)
    dk = c * np.outer(ds, q)
    return o, m + math.log(z), dq, dk, dv


def row_weights(q: np.ndarray, keys: np.ndarray, values: np.ndarray, do: np.ndarray):
    """The softmax weights p and score gradients ds of one row (the same
    quantities attend_grad forms), for bounding rounding effects in tests."""
    c = 1.0 / math.sqrt(q.shape[-1])
    s = c * (keys @ q)
    e = np.exp(s - s.max())
    p = e / e.sum()
    dp = values @ do
    return p, p * (dp - float(p @ dp))


def attention_grads(q_cube, k_cube, v_cube, g: Geometry, sel_video: dict, dout_raster,
                    q_extra=None, sel_extra=None, dout_extra=None, head_map=None, k_text=None, v_text=None):
    """Gradients of every row in ``sel_video`` ({(hq, pos): cubes}) and
    ``sel_extra`` ({(hq, m): cubes}; extra rows attend their selected cubes,
    and, with ``k_text`` / ``v_text`` [n_text][Hkv][d] given, text keys 0..m
    as well: a text prefill, where text row m attends the text tokens up to
    itself).  Cube-layout inputs as from ``partition``; dout_raster [N][Hq][d]
    (raster order), dout_extra [n_extra][Hq][d].

    Returns dict with float64 arrays: dq_raster [N][Hq][d] (rows not listed
    are zero), dk_raster / dv_raster [N][Hkv][d], dq_extra [n_extra][Hq][d],
    dk_text / dv_text [n_text][Hkv][d] (with text keys),
    lse {(kind, hq, row): value}, o {(kind, hq, row): [d]}."""
    Hq, N, d = q_cube.shape
    Hkv = k_cube.shape[0]
    S = g.S
    n_all = np.arange(g.N)
    cube, r = cube_coords(g, n_all)
    raster_of_pos = np.empty(g.N, dtype=np.int64)
    raster_of_pos[cube * S + r] = n_all
    dq = np.zeros((g.N, Hq, d))
    dk = np.zeros((g.N, Hkv, d))
    dv = np.zeros((g.N, Hkv, d))
    n_extra = 0 if q_extra is None else q_extra.shape[0]
    dqx = np.zeros((n_extra, Hq, d))
    n_text = 0 if k_text is None else k_text.shape[0]
    dkt = np.zeros((n_text, Hkv, d))
    dvt = np.zeros((n_text, Hkv, d))
    lse, outs = {}, {}

    def run(kind, hq, row, qv, dov, cubes, n_tk=0):
        """n_tk: text keys 0 .. n_tk - 1 join the row's keys after its cubes."""
        kv = _kv_head(hq, Hq, Hkv, head_map)
        pos = np.concatenate([np.arange(j * S, (j + 1) * S) for j in cubes]) if cubes else np.zeros(0, np.int64)
        keys = to_f64(k_cube[kv][pos])
        vals = to_f64(v_cube[kv][pos])
        if n_tk:
            keys = np.concatenate([keys, to_f64(k_text[:n_tk, kv])])
            vals = np.concatenate([vals, to_f64(v_text[:n_tk, kv])])
        o, l, gq, gk, gv = attend_grad(qv, keys, vals, dov)
        nv = len(pos)
        ras = raster_of_pos[pos]
        np.add.at(dk[:, kv], ras, gk[:nv])
        np.add.at(dv[:, kv], ras, gv[:nv])
        if n_tk:
            dkt[:n_tk, kv] += gk[nv:]
            dvt[:n_tk, kv] += gv[nv:]
        lse[(kind, hq, row)] = l
        outs[(kind, hq, row)] = o
        return gq

    for (hq, p), cubes in sel_video.items():
        c = p // S
        allc = sorted(set(int(j) for j in cubes) | {c})
        n = raster_of_pos[p]
        dq[n, hq] = run("v", hq, p, to_f64(q_cube[hq, p]), to_f64(dout_raster[n, hq]), allc)
    for (hq, m), cubes in (sel_extra or {}).items():
        dqx[m, hq] = run("x", hq, m, to_f64(q_extra[m, hq]), to_f64(dout_extra[m, hq]),
                         [int(j) for j in cubes], m + 1 if n_text else 0)
    return {"dq_raster": dq, "dk_raster": dk, "dv_raster": dv, "dq_extra": dqx, "dk_text": dkt, "dv_text": dvt,
            "lse": lse, "o": outs}

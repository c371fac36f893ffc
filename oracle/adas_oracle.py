"""CPU oracle for AdaS-Attn (adaptive cube-selective attention).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module never
calls the product path: the two share no code, only the seeded inputs from
``workloads``.

Everything is plain NumPy in float64, written from the method's description:

* AdaSpark page on papernotes.org, "关键设计" (key designs):
  item 1 (3D spatio-temporal cube partition: h x w x t windows, the cube is
  the atomic unit of selection), item 2 (AdaS-Attn: score each query against
  the mean key of every preceding cube, softmax with 1/sqrt(d_k), keep the
  Top-p (nucleus) set S_i, always keep full attention to the own cube),
  item 4 (one threshold p).
* thelatestinai.com listing of the same paper: Figure 2 caption (each token
  query selects over preceding cubes), Tables 3 and 5 (cube shapes).

Readings where the pages leave a step open (each is also listed with the
design notes of the repository):

* P_i's index i is the query's *cube*; "preceding" means cubes 0..c-1.
* Cubes are numbered in raster order of their first token:
  c = ((f // t) * nH + y // h) * nW + x // w; inside a cube tokens keep
  raster order: r = ((f % t) * h + y % h) * w + x % w.
* Own-cube attention is bidirectional over all S tokens of the cube (block
  causal); the own cube is not part of the selection softmax.
* Top-p: order cubes by (P descending, index ascending), take the shortest
  prefix whose sequential float64 sum reaches p (>= p); p >= 1 keeps all.
  The selected set is emitted in ascending cube order.
* Attention over the union of selected cubes and the own cube is one exact
  softmax with scale 1/sqrt(d_k); no gating, no re-weighting by P.
* Text queries select over all video cubes and attend causally to text
  tokens 0..m (when text K/V exist); decode queries select over all cubes
  and attend to the selected cubes only.

Inputs: bf16 tensors arrive as uint16 bit patterns, f32 as float32; both are
converted exactly to float64 here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Geometry", "to_f64", "cube_coords", "partition", "mean_keys",
    "kbar_to_f32", "selection_logits", "softmax", "selection_probabilities",
    "top_p", "top_k", "top_p_batch", "select_video_rows", "select_extra_rows",
    "attend", "attention_video_row", "attention_extra_row",
    "attention_video_rows", "dense_block_causal",
]


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------
def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a bf16 bit array (uint16) or a float32 array."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    if x.dtype == np.float64:
        return x
    raise TypeError(f"unsupported input dtype {x.dtype}")


# ---------------------------------------------------------------------------
# O1: cube partition (key design 1)
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    """Frame grid T x H x W tokens, cube extents ct (time), ch, cw."""
    T: int
    H: int
    W: int
    ct: int
    ch: int
    cw: int

    def __post_init__(self):
        if self.T % self.ct or self.H % self.ch or self.W % self.cw:
            raise ValueError("cube extents must divide the frame grid")

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def S(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def nT(self) -> int:
        return self.T // self.ct

    @property
    def nH(self) -> int:
        return self.H // self.ch

    @property
    def nW(self) -> int:
        return self.W // self.cw

    @property
    def n_cubes(self) -> int:
        return self.nT * self.nH * self.nW

    @classmethod
    def of(cls, wl) -> "Geometry":
        return cls(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw)


def cube_coords(g: Geometry, n):
    """Raster token n = (f*H + y)*W + x  ->  (cube index c, offset r in cube)."""
    n = np.asarray(n, dtype=np.int64)
    f = n // (g.H * g.W)
    y = (n // g.W) % g.H
    x = n % g.W
    c = ((f // g.ct) * g.nH + y // g.ch) * g.nW + x // g.cw
    r = ((f % g.ct) * g.ch + y % g.ch) * g.cw + x % g.cw
    return c, r


def partition(x_raster: np.ndarray, g: Geometry):
    """Cube-contiguous, head-major copy of a token-major tensor.

    x_raster: [N][nh][d] (any dtype; values are copied bit for bit).
    Returns (x_cube [nh][N][d], perm [N] int32) with
    x_cube[h][c*S + r] = x_raster[n][h] and perm[c*S + r] = n.
    """
    N = g.N
    if x_raster.shape[0] != N:
        raise ValueError("token count does not match the grid")
    n = np.arange(N, dtype=np.int64)
    c, r = cube_coords(g, n)
    pos = c * g.S + r
    perm = np.empty(N, dtype=np.int32)
    perm[pos] = n
    x_cube = np.empty((x_raster.shape[1], N, x_raster.shape[2]), dtype=x_raster.dtype)
    x_cube[:, pos, :] = np.swapaxes(x_raster, 0, 1)
    return x_cube, perm


# ---------------------------------------------------------------------------
# O2: cube mean keys (key design 2: k-bar_j)
# ---------------------------------------------------------------------------
def mean_keys(k_cube: np.ndarray, g: Geometry) -> np.ndarray:
    """kbar[h][j] = (1/S) * sum of the S keys of cube j, in float64.

    k_cube: [Hkv][N][d] cube layout (as produced by ``partition``)."""
    k = to_f64(k_cube)
    Hkv, N, d = k.shape
    return k.reshape(Hkv, g.n_cubes, g.S, d).sum(axis=2) / g.S


def kbar_to_f32(kbar: np.ndarray) -> np.ndarray:
    """The float32 value the library reports: round-to-nearest-even."""
    return kbar.astype(np.float32)


# ---------------------------------------------------------------------------
# O3/O4: selection softmax P_i (key design 2, the P_i equation)
# ---------------------------------------------------------------------------
def selection_logits(q: np.ndarray, kbar_prev: np.ndarray) -> np.ndarray:
    """z_j = q . kbar_j / sqrt(d_k) for the candidate cubes (rows of kbar_prev).

    q: [..., d] float64, kbar_prev: [n, d] float64 -> [..., n]."""
    d = q.shape[-1]
    return (q @ kbar_prev.T) / math.sqrt(d)


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax along the last axis, max-subtracted."""
    if z.shape[-1] == 0:
        return z.copy()
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def selection_probabilities(q: np.ndarray, kbar_prev: np.ndarray) -> np.ndarray:
    return softmax(selection_logits(q, kbar_prev))


# ---------------------------------------------------------------------------
# O5: Top-p (nucleus) cube set S_i
# ---------------------------------------------------------------------------
def top_p(P: np.ndarray, p: float) -> np.ndarray:
    """Smallest prefix of cubes ordered by (P desc, index asc) whose
    sequential float64 sum reaches p; returned in ascending cube order.

    Empty candidate list -> empty set; p >= 1 -> every candidate (a float sum
    may fall short of exactly 1); if rounding leaves the full sum below p the
    whole list is kept."""
    n = len(P)
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    if p >= 1.0:
        return np.arange(n, dtype=np.int32)
    order = np.lexsort((np.arange(n), -P))      # primary: -P ascending; ties: index ascending
    total = 0.0
    k = n
    for m, j in enumerate(order):
        total += float(P[j])
        if total >= p:
            k = m + 1
            break
    return np.sort(order[:k]).astype(np.int32)


def top_k(P: np.ndarray, k: int) -> np.ndarray:
    """The fixed-budget alternative the AdaSpark listing compares Top-p with
    (thelatestinai.com listing, Table 4, "Top-K" row): the k cubes of largest
    P, equal P taken lower index first (the same order as Top-p), returned in
    ascending cube order; fewer than k candidates -> all of them."""
    n = len(P)
    if k < 1:
        raise ValueError("k must be >= 1")
    order = np.lexsort((np.arange(n), -P))      # -P ascending, then index ascending
    return np.sort(order[:min(k, n)]).astype(np.int32)


def top_p_batch(P: np.ndarray, p: float):
    """``top_p`` applied to every row of P [rows][n] (same n for all rows).

    Returns (counts [rows] int32, mask [rows][n] bool); row r's set is
    ``np.nonzero(mask[r])[0]`` (ascending)."""
    rows, n = P.shape
    if n == 0:
        return np.zeros(rows, np.int32), np.zeros((rows, 0), bool)
    if p >= 1.0:
        return np.full(rows, n, np.int32), np.ones((rows, n), bool)
    order = np.argsort(-P, axis=1, kind="stable")           # ties keep ascending index
    cum = np.cumsum(np.take_along_axis(P, order, axis=1), axis=1)  # sequential sums
    reached = cum >= p
    k = np.where(reached.any(axis=1), reached.argmax(axis=1) + 1, n)
    rank = np.empty_like(order)
    np.put_along_axis(rank, order, np.arange(n)[None, :].repeat(rows, 0), axis=1)
    mask = rank < k[:, None]
    return k.astype(np.int32), mask


# ---------------------------------------------------------------------------
# selection over whole row sets
# ---------------------------------------------------------------------------
def _kv_head(hq: int, Hq: int, Hkv: int, head_map=None) -> int:
    if head_map is not None:
        return int(head_map[hq])
    return hq // (Hq // Hkv)


def select_video_rows(q_cube, kbar, g: Geometry, p: float, heads=None,
                      cubes=None, head_map=None, k=None):
    """Top-p sets of video rows (Top-k sets when k is given).

    q_cube: [Hq][N][d] cube layout; kbar: [Hkv][Nc][d] float64.
    Returns {(hq, pos): ascending int32 array} for the requested heads and
    query cubes (default: all)."""
    Hq = q_cube.shape[0]
    Hkv = kbar.shape[0]
    heads = range(Hq) if heads is None else heads
    cubes = range(g.n_cubes) if cubes is None else cubes
    out = {}
    for hq in heads:
        kb = kbar[_kv_head(hq, Hq, Hkv, head_map)]
        for c in cubes:
            q = to_f64(q_cube[hq, c * g.S:(c + 1) * g.S])
            P = selection_probabilities(q, kb[:c])
            if k is not None:
                for r in range(g.S):
                    out[(hq, c * g.S + r)] = top_k(P[r], k)
                continue
            _, mask = top_p_batch(P, p)
            for r in range(g.S):
                out[(hq, c * g.S + r)] = np.nonzero(mask[r])[0].astype(np.int32)
    return out


def select_extra_rows(q_extra, kbar, p: float, rows=None, head_map=None, k=None):
    """Top-p sets of text / decode rows (every video cube is a candidate;
    Top-k sets when k is given).

    q_extra: [Nt][Hq][d]. Returns {(hq, m): ascending int32 array}."""
    Nt, Hq, _ = q_extra.shape
    Hkv = kbar.shape[0]
    rows = range(Nt) if rows is None else rows
    out = {}
    for hq in range(Hq):
        kb = kbar[_kv_head(hq, Hq, Hkv, head_map)]
        idx = list(rows)
        if not idx:
            continue
        q = to_f64(q_extra[idx, hq])
        P = selection_probabilities(q, kb)
        if k is not None:
            for i, m in enumerate(idx):
                out[(hq, m)] = top_k(P[i], k)
            continue
        _, mask = top_p_batch(P, p)
        for i, m in enumerate(idx):
            out[(hq, m)] = np.nonzero(mask[i])[0].astype(np.int32)
    return out


# ---------------------------------------------------------------------------
# O6: attention over the selected cubes plus the own cube
# ---------------------------------------------------------------------------
def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Exact softmax attention of one query over a key/value set (float64)."""
    s = keys @ q / math.sqrt(q.shape[-1])
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ values


def _cube_tokens(x_cube_h: np.ndarray, cubes, S: int) -> np.ndarray:
    return np.concatenate([x_cube_h[j * S:(j + 1) * S] for j in cubes], axis=0)


def attention_video_row(q_cube, k_cube, v_cube, g: Geometry, hq: int, pos: int,
                        sel: np.ndarray, head_map=None) -> np.ndarray:
    """Output of video row (hq, pos): attention over selected cubes and the
    row's own cube (all its S tokens)."""
    Hq, Hkv = q_cube.shape[0], k_cube.shape[0]
    kv = _kv_head(hq, Hq, Hkv, head_map)
    c = pos // g.S
    cubes = sorted(set(int(j) for j in sel) | {c})
    keys = to_f64(_cube_tokens(k_cube[kv], cubes, g.S))
    vals = to_f64(_cube_tokens(v_cube[kv], cubes, g.S))
    return attend(to_f64(q_cube[hq, pos]), keys, vals)


def attention_extra_row(q_extra, k_cube, v_cube, g: Geometry, hq: int, m: int,
                        sel: np.ndarray, k_text=None, v_text=None,
                        head_map=None) -> np.ndarray:
    """Output of text / decode row (hq, m): the selected video cubes plus,
    when text K/V are given, text tokens 0..m (causal)."""
    Hq, Hkv = q_extra.shape[1], k_cube.shape[0]
    kv = _kv_head(hq, Hq, Hkv, head_map)
    cubes = [int(j) for j in sel]
    parts_k, parts_v = [], []
    if cubes:
        parts_k.append(to_f64(_cube_tokens(k_cube[kv], cubes, g.S)))
        parts_v.append(to_f64(_cube_tokens(v_cube[kv], cubes, g.S)))
    if k_text is not None:
        parts_k.append(to_f64(k_text[: m + 1, kv]))
        parts_v.append(to_f64(v_text[: m + 1, kv]))
    keys = np.concatenate(parts_k, axis=0)
    vals = np.concatenate(parts_v, axis=0)
    return attend(to_f64(q_extra[m, hq]), keys, vals)


def attention_video_rows(q_cube, k_cube, v_cube, g: Geometry, sel: dict,
                         head_map=None) -> dict:
    """{(hq, pos): output} for every (hq, pos) key of ``sel``."""
    return {key: attention_video_row(q_cube, k_cube, v_cube, g, key[0], key[1], s, head_map)
            for key, s in sel.items()}


# ---------------------------------------------------------------------------
# dense block-causal attention: what p = 1 must reduce to
# ---------------------------------------------------------------------------
def dense_block_causal(q_raster, k_raster, v_raster, g: Geometry, head_map=None):
    """Dense masked attention in raster order: token i sees token k iff
    cube(k) <= cube(i).  Returns [N][Hq][d] float64.

    Built from a dense N x N mask, with no gathering, so that it is an
    independent route to the p = 1 result."""
    q = to_f64(q_raster)
    k = to_f64(k_raster)
    v = to_f64(v_raster)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    cube, _ = cube_coords(g, np.arange(N))
    allowed = cube[None, :] <= cube[:, None]
    out = np.empty_like(q)
    for hq in range(Hq):
        kv = _kv_head(hq, Hq, Hkv, head_map)
        s = (q[:, hq] @ k[:, kv].T) / math.sqrt(d)
        s = np.where(allowed, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[:, hq] = w @ v[:, kv]
    return out

"""CPU oracle for AdaS-FFN (adaptive token-selective FFN).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It never calls
the HIP library or its binding; the two share only the seeded inputs of
``workloads``.

Plain NumPy in float64, written from the method's description:

* AdaSpark page on papernotes.org, "关键设计" item 3 (AdaS-FFN): each video
  token's importance is estimated from its L2 norm; Top-p picks the tokens
  that go through the FFN; a skipped token k of cube i gets
  y_k = x_k + m_i, where m_i is the mean of FFN(x_j) over the active set M_i
  of that cube; text tokens always go through the FFN.  Item 4: the same
  Top-p rule and the same threshold p as AdaS-Attn.
* thelatestinai.com listing of the same paper: Figure 2 caption (tokens are
  selected *within each cube*; mean compensation for the rest; text dense),
  Figure 4 (keep ratio per cube), Table 5 (Qwen2.5-VL backbones, whose MLP
  is SwiGLU).

Readings where the pages leave a step open (each is also listed with the
design notes of the repository):

* The Top-p distribution over the S tokens of a cube is each token's share of
  the cube's summed L2 norm, P_r = ||x_r|| / sum_j ||x_j||.  The set is the
  shortest prefix of tokens ordered by (P descending, offset ascending) whose
  sequential float64 sum reaches p (the AdaS-Attn rule); p >= 1 keeps all.
* Active tokens get the usual residual FFN output y = x + FFN(x); the
  compensation formula is the skipped tokens' counterpart of it.
* FFN(x) = W_down (silu(W_gate x) * (W_up x)), silu(t) = t / (1 + e^-t),
  with the weights in the nn.Linear [out][in] layout.  Any normalisation a
  model applies before its MLP is outside the formula and not modelled.
* Norms are taken on the FFN input x itself.

Inputs arrive as bf16 bit patterns (uint16) and are converted exactly.
"""
from __future__ import annotations

import math

import numpy as np

from .adas_oracle import Geometry, cube_coords, to_f64, top_p

__all__ = [
    "token_norms", "norm_shares", "select_tokens", "cube_tokens", "silu", "swiglu_ffn",
    "ffn_select", "adas_ffn_cubes", "adas_ffn_text",
]


def token_norms(x: np.ndarray) -> np.ndarray:
    """L2 norm of every row of x ([..., hidden]) in float64."""
    x = to_f64(x)
    return np.sqrt(np.sum(x * x, axis=-1))


def norm_shares(norms: np.ndarray) -> np.ndarray:
    """Each token's share of the cube's summed norm (a probability vector).
    The total is summed in index order.  An all-zero cube is uniform."""
    total = 0.0
    for v in norms:
        total += float(v)
    if total == 0.0:
        return np.full(len(norms), 1.0 / len(norms))
    return np.asarray(norms, dtype=np.float64) / total


def select_tokens(norms: np.ndarray, p: float) -> np.ndarray:
    """Active offsets of one cube (ascending): Top-p over the norm shares."""
    return top_p(norm_shares(norms), p)


def cube_tokens(g: Geometry, c: int) -> np.ndarray:
    """Raster indices of the S tokens of cube c, in offset order r = 0..S-1."""
    n = np.arange(g.N, dtype=np.int64)
    cc, r = cube_coords(g, n)
    sel = np.nonzero(cc == c)[0]
    out = np.empty(g.S, dtype=np.int64)
    out[r[sel]] = sel
    return out


def silu(t: np.ndarray) -> np.ndarray:
    return t / (1.0 + np.exp(-t))


def swiglu_ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """FFN(x) = W_down (silu(W_gate x) * (W_up x)) for every row of x ([M][hidden]),
    float64; weights in the [out][in] layout (bf16 bits or float arrays)."""
    x = to_f64(x)
    g = x @ to_f64(w_gate).T
    u = x @ to_f64(w_up).T
    return (silu(g) * u) @ to_f64(w_down).T


def ffn_select(x: np.ndarray, g: Geometry, p: float, cubes=None) -> dict:
    """{cube c: (raster ids of its tokens in offset order, active offsets ascending)}."""
    cubes = range(g.n_cubes) if cubes is None else cubes
    out = {}
    for c in cubes:
        toks = cube_tokens(g, c)
        out[c] = (toks, select_tokens(token_norms(x[toks]), p))
    return out


def adas_ffn_cubes(x, g: Geometry, p: float, w_gate, w_up, w_down, cubes=None,
                   weights64=None) -> dict:
    """Outputs y of the tokens of the given cubes.

    Returns {c: (raster ids, active offsets, y [S][hidden] float64)}: active
    tokens y = x + FFN(x); skipped tokens y = x + mean of FFN over the active
    tokens of the same cube.  ``weights64`` may hold the three weights already
    converted to float64 (the same values; saves the conversion per call)."""
    if weights64 is not None:
        w_gate, w_up, w_down = weights64
    out = {}
    for c, (toks, act) in ffn_select(x, g, p, cubes).items():
        xc = to_f64(x[toks])
        f_act = swiglu_ffn(xc[act], w_gate, w_up, w_down)
        y = xc.copy()
        y[act] += f_act
        skipped = np.setdiff1d(np.arange(g.S), act)
        if len(skipped):
            m = f_act.sum(axis=0) / len(act)
            y[skipped] += m
        out[c] = (toks, act, y)
    return out


def adas_ffn_text(x_text, w_gate, w_up, w_down, rows=None) -> np.ndarray:
    """Text tokens go through the FFN densely: y = x + FFN(x)."""
    xt = to_f64(x_text) if rows is None else to_f64(x_text[rows])
    return xt + swiglu_ffn(xt, w_gate, w_up, w_down)

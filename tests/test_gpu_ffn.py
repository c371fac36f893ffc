"""GPU parity of AdaS-FFN (include/adas_ffn.h) against the float64 oracle
(oracle/ffn_oracle.py), through the C ABI binding.

Bars:
  * token selection (counts, masks, offsets, compact rows): exact.  Both
    sides take the decision in float64 from the same bf16 bits; a row may
    differ only if the oracle's running sum at the cut lies within 1e-12 of p
    (counted; none expected).
  * outputs: y is bf16, whose unit roundoff is u = 2^-8 (8 significant
    bits).  Its error against float64 scales with the size of the token's
    output row, not of the single element (FFN(x) may nearly cancel x in one
    element): the final rounding of y (at most u |y|, and |y| reaches 4-5
    rms(y) in a row of ~Gaussian entries: <= 1.95e-2 rms); the bf16 rounding
    of the hidden activation before W_down (relative error up to u per
    element with independent signs, so about u/sqrt(3) = 2.3e-3 rms(FFN) per
    output, <= 1.35e-2 rms at 6 sigma); float32 accumulation (~1e-6,
    negligible).  Both extremes in one element are not expected together.
    With e = |y_dev - y_ref| / max(1, rms of the token's y_ref row) the bars
    are max e <= 3e-2 and mean e <= 3e-3 (mean final rounding about
    u/4 E|y| / rms ~ 0.8e-3 to 1.1e-3, plus mean hidden-rounding error
    0.8 u/sqrt(3) ~ 1.8e-3).
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import adas_oracle as O
from oracle import ffn_oracle as F
from tests.gpu_harness import bits, log, to_dev

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 3e-2, 3e-3


def _geom(wl):
    from adaptive_cube_sparse_amd import FfnGeometry
    return FfnGeometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.hidden, wl.inter)


def _run(wl, data, p=None, dev="cuda:0"):
    from adaptive_cube_sparse_amd import AdasFFN
    layer = AdasFFN(_geom(wl), wl.p if p is None else p, to_dev(data["w_gate"], dev), to_dev(data["w_up"], dev),
                    to_dev(data["w_down"], dev), n_text=wl.n_text, device=dev)
    xt = to_dev(data["x_text"], dev) if wl.n_text else None
    layer.forward(to_dev(data["x"], dev), xt)
    torch.cuda.synchronize()
    return layer


def _og(wl):
    return O.Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw)


def _check_selection(wl, data, layer, p):
    """Exact selection of every cube; returns the oracle's {c: (toks, act)}."""
    g = _og(wl)
    norms = F.token_norms(data["x"])
    counts = layer.act_count.cpu().numpy()
    masks = layer.act_mask.cpu().numpy().view(np.uint32)
    off = layer.act_off.cpu().numpy()
    rows = layer.act_rows.cpu().numpy()
    sel, near = {}, 0
    for c in range(g.n_cubes):
        toks = F.cube_tokens(g, c)
        act = F.select_tokens(norms[toks], p)
        sel[c] = (toks, act)
        got = np.array([r for r in range(g.S) if (masks[c, r // 32] >> (r % 32)) & 1])
        if got.tolist() != act.tolist() or counts[c] != len(act):
            P = F.norm_shares(norms[toks])
            cum = np.cumsum(np.sort(P)[::-1])
            k = len(act)
            if min(abs(cum[k - 1] - p), abs(cum[k - 2] - p) if k >= 2 else 1.0) <= 1e-12:
                near += 1
                continue
            raise AssertionError(f"cube {c}: device {got.tolist()} oracle {act.tolist()}")
    want_off = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(off, want_off), "act_off is not the prefix sum of act_count"
    for c in range(g.n_cubes):
        toks = F.cube_tokens(g, c)
        got = [r for r in range(g.S) if (masks[c, r // 32] >> (r % 32)) & 1]
        assert rows[off[c]:off[c + 1]].tolist() == toks[got].tolist(), f"act_rows of cube {c}"
    log(f"  selection: {g.n_cubes} cubes exact ({near} near-threshold), keep ratio "
        f"{counts.sum() / g.N:.3f}")
    assert near <= max(1, g.n_cubes // 1000)
    return sel


def _err(got_bits, ref):
    got = O.to_f64(got_bits)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return np.abs(got - ref) / np.maximum(1.0, rms)


def _check_outputs(wl, data, layer, p, cubes, text_rows=None):
    g = _og(wl)
    w64 = (O.to_f64(data["w_gate"]), O.to_f64(data["w_up"]), O.to_f64(data["w_down"]))
    y = bits(layer.y)
    errs = []
    for c, (toks, act, yref) in F.adas_ffn_cubes(data["x"], g, p, None, None, None, cubes=cubes,
                                                 weights64=w64).items():
        errs.append(_err(y[toks], yref).ravel())
    if wl.n_text:
        rows = np.arange(wl.n_text) if text_rows is None else np.asarray(text_rows)
        yt = bits(layer.y_text)
        ref = F.adas_ffn_text(data["x_text"], *w64, rows=rows)
        errs.append(_err(yt[rows], ref).ravel())
    e = np.concatenate(errs)
    log(f"  outputs: {e.size} values, max e {e.max():.3e}, mean e {e.mean():.3e} "
        f"(bars {TOL_MAX}, {TOL_MEAN})")
    assert np.all(np.isfinite(e))
    assert e.max() <= TOL_MAX and e.mean() <= TOL_MEAN


def _case(wl, p=None, cubes=None, text_rows=None):
    p = wl.p if p is None else p
    log(f"[ffn] {wl.name} grid {wl.T}x{wl.H}x{wl.W} cube ({wl.ct},{wl.ch},{wl.cw}) hidden {wl.hidden} "
        f"inter {wl.inter} text {wl.n_text} p {p}")
    data = workloads.generate_ffn(wl)
    layer = _run(wl, data, p)
    _check_selection(wl, data, layer, p)
    g = _og(wl)
    _check_outputs(wl, data, layer, p, range(g.n_cubes) if cubes is None else cubes, text_rows)
    return layer, data


def test_ffn_tiny_every_token():
    _case(workloads.get_ffn("ffn_tiny"))


@pytest.mark.parametrize("p", [1.0, 1e-9, 0.5])
def test_ffn_tiny_p_extremes(p):
    # p = 1: dense FFN on every token; p -> 0: one token per cube, all others
    # take its FFN output
    _case(workloads.get_ffn("ffn_tiny").replace(name=f"ffn_tiny_p{p}"), p=p)


def test_ffn_cube_of_128_with_text_and_ragged_tiles():
    # S = 128 (four mask words), 16 cubes, 70 text rows: the row count is not a
    # multiple of the 256-row tile, and text rows share the last tile with video rows
    wl = workloads.FfnWorkload(name="ffn_s128", T=8, H=16, W=16, ct=2, ch=8, cw=8, hidden=512, inter=768,
                               p=0.8, seed=2101, n_text=70)
    _case(wl)


def test_ffn_several_column_tiles_and_k_stages():
    # hidden 1024 (4 down-projection column tiles), inter 1280 (10 gate/up tiles,
    # 20 stages of the down projection), 1024 tokens in 16 cubes of 64
    wl = workloads.FfnWorkload(name="ffn_mid", T=4, H=16, W=16, ct=4, ch=4, cw=4, hidden=1024, inter=1280,
                               p=0.7, seed=2102)
    _case(wl)


def test_ffn3b_full_size_every_token():
    # the 3B-shaped layer bench.py times: every token of all 256 cubes
    _case(workloads.get_ffn("ffn3b"))


def test_ffn7b_full_size_every_token():
    # the 7B-shaped layer bench.py times: every token of every cube
    _case(workloads.get_ffn("ffn7b"))


def test_ffn_deterministic():
    wl = workloads.get_ffn("ffn_tiny")
    data = workloads.generate_ffn(wl)
    a = bits(_run(wl, data).y).copy()
    b = bits(_run(wl, data).y)
    assert np.array_equal(a, b)

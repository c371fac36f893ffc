"""Pins of the AdaS-FFN oracle (oracle/ffn_oracle.py) against what the method
and the mathematics fix, independently of the oracle's own code paths.

Method: AdaSpark, papernotes.org, key design 3 (L2-norm importance, Top-p per
cube, mean compensation y_k = x_k + m_i for skipped tokens, text dense) and
key design 4 (the shared Top-p rule)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import adas_oracle as O
from oracle import ffn_oracle as F

from conftest import GOLDEN


def _bf16(x):
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_golden_identity_weights():
    case = json.load(open(os.path.join(GOLDEN, "ffn_cases.json")))
    gd = case["grid"]
    g = O.Geometry(gd["T"], gd["H"], gd["W"], gd["ct"], gd["ch"], gd["cw"])
    x = np.asarray(case["x"], dtype=np.float64)
    eye = np.eye(2)
    for cs in case["cases"]:
        out = F.adas_ffn_cubes(x, g, cs["p"], eye, eye, eye)
        toks, act, y = out[0]
        assert toks.tolist() == [0, 1, 2, 3]
        assert act.tolist() == cs["active"], (cs["p"], act)
        np.testing.assert_allclose(y, np.asarray(cs["y"]), rtol=0, atol=1e-13)


def _brute_force_tokens(norms, p):
    """Fewest tokens whose share reaches p; among those the largest mass; then
    the lexicographically smallest offsets in descending-P order (tie rule)."""
    n = len(norms)
    P = np.asarray(norms) / sum(norms)
    for k in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), k):
            m = sum(P[j] for j in sub)
            if m >= p - 1e-12:
                key = (-round(m, 12), sorted(sub))
                if best is None or key < best[0]:
                    best = (key, sub)
        if best is not None:
            return sorted(best[1])
    return list(range(n))


def test_token_selection_matches_subset_enumeration():
    rng = np.random.default_rng(7)
    for trial in range(300):
        n = int(rng.integers(1, 10))
        norms = rng.choice([1.0, 2.0, 3.0, 5.0, 0.5], size=n) if trial % 3 == 0 else rng.random(n) + 0.01
        p = float(rng.choice([0.1, 0.3, 0.5, 0.7, 0.9, 0.95]))
        got = F.select_tokens(np.asarray(norms), p).tolist()
        want = _brute_force_tokens(norms, p)
        # ties of equal mass at the cut: the oracle takes the lower offsets
        assert got == want or (len(got) == len(want)
                               and abs(sum(np.asarray(norms)[got]) - sum(np.asarray(norms)[want])) < 1e-12), \
            (norms, p, got, want)


def test_equal_norms_take_the_lowest_offsets():
    # rows that are signed permutations of one bf16 vector have bit-identical norms
    rng = np.random.default_rng(3)
    base = workloads.bf16_bits_to_f32(_bf16(rng.standard_normal(16))).astype(np.float64)
    S = 10
    rows = np.stack([np.roll(base, k) * (-1) ** k for k in range(S)])
    norms = F.token_norms(rows)
    assert len(set(norms.tolist())) == 1
    for p in (0.05, 0.33, 0.65, 0.91):
        assert F.select_tokens(norms, p).tolist() == list(range(math.ceil(p * S))), p


def test_selection_is_scale_invariant_and_monotone():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 64)) * np.exp(rng.standard_normal(32))[:, None]
    n = F.token_norms(x)
    for p in (0.3, 0.7, 0.9):
        a = F.select_tokens(n, p)
        assert F.select_tokens(F.token_norms(4.0 * x), p).tolist() == a.tolist()
        # the kept tokens are the largest ones: every kept norm >= every skipped norm
        rest = np.setdiff1d(np.arange(32), a)
        if len(rest):
            assert n[a].min() >= n[rest].max()
        # minimality and reach
        P = n / n.sum()
        assert P[a].sum() >= p and P[a].sum() - P[a].min() < p
    # nested in p
    prev = set()
    for p in np.linspace(0.05, 1.0, 20):
        cur = set(F.select_tokens(n, float(p)).tolist())
        assert prev <= cur
        prev = cur


def _torch_swiglu(x, wg, wu, wd):
    xt = torch.from_numpy(x)
    g = torch.nn.functional.linear(xt, torch.from_numpy(wg))
    u = torch.nn.functional.linear(xt, torch.from_numpy(wu))
    return torch.nn.functional.linear(torch.nn.functional.silu(g) * u, torch.from_numpy(wd)).numpy()


def test_swiglu_matches_torch_and_a_scalar_closed_form():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, 48))
    wg, wu, wd = rng.standard_normal((80, 48)), rng.standard_normal((80, 48)), rng.standard_normal((48, 80))
    np.testing.assert_allclose(F.swiglu_ffn(x, wg, wu, wd), _torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-10)
    # hidden = inter = 1: FFN(x) = wd * silu(wg x) * (wu x)
    got = F.swiglu_ffn(np.array([[1.5]]), np.array([[2.0]]), np.array([[-0.5]]), np.array([[3.0]]))
    want = 3.0 * (3.0 / (1.0 + math.exp(-3.0))) * (-0.75)
    assert abs(got[0, 0] - want) < 1e-14


def _grid():
    return O.Geometry(4, 4, 4, 2, 2, 2)    # 8 cubes of 8 tokens


def test_cube_tokens_by_enumeration():
    g = _grid()
    for c in range(g.n_cubes):
        bt, rem = divmod(c, g.nH * g.nW)
        by, bx = divmod(rem, g.nW)
        want = [((bt * g.ct + dt) * g.H + by * g.ch + dy) * g.W + bx * g.cw + dx
                for dt in range(g.ct) for dy in range(g.ch) for dx in range(g.cw)]
        assert F.cube_tokens(g, c).tolist() == want


def test_compensation_uses_the_own_cube_and_the_linear_route():
    g = _grid()
    rng = np.random.default_rng(2)
    hidden, inter = 32, 48
    x = rng.standard_normal((g.N, hidden)) * np.exp(rng.standard_normal(g.N))[:, None]
    wg, wu, wd = (rng.standard_normal((inter, hidden)), rng.standard_normal((inter, hidden)),
                  rng.standard_normal((hidden, inter)))
    out = F.adas_ffn_cubes(x, g, 0.6, wg, wu, wd)
    for c, (toks, act, y) in out.items():
        skipped = np.setdiff1d(np.arange(g.S), act)
        assert 1 <= len(act) <= g.S
        # active tokens: the residual FFN of their own state (torch route)
        np.testing.assert_allclose(y[act], x[toks[act]] + _torch_swiglu(x[toks[act]], wg, wu, wd),
                                   rtol=1e-12, atol=1e-10)
        if len(skipped):
            # every skipped token moves by the same vector ...
            d = y[skipped] - x[toks[skipped]]
            np.testing.assert_allclose(d, np.broadcast_to(d[0], d.shape), rtol=0, atol=1e-12)
            # ... which is W_down applied to the mean hidden activation of the
            # cube's active tokens (linearity of the last projection)
            xa = torch.from_numpy(x[toks[act]])
            h = torch.nn.functional.silu(xa @ torch.from_numpy(wg).T) * (xa @ torch.from_numpy(wu).T)
            m = (h.mean(dim=0) @ torch.from_numpy(wd).T).numpy()
            np.testing.assert_allclose(d[0], m, rtol=1e-11, atol=1e-10)


def test_p_one_is_the_dense_ffn_and_tiny_p_keeps_the_largest_token():
    g = _grid()
    rng = np.random.default_rng(9)
    hidden, inter = 16, 24
    x = rng.standard_normal((g.N, hidden)) * np.exp(rng.standard_normal(g.N))[:, None]
    wg, wu, wd = (rng.standard_normal((inter, hidden)), rng.standard_normal((inter, hidden)),
                  rng.standard_normal((hidden, inter)))
    dense = x + _torch_swiglu(x, wg, wu, wd)
    for c, (toks, act, y) in F.adas_ffn_cubes(x, g, 1.0, wg, wu, wd).items():
        assert act.tolist() == list(range(g.S))
        np.testing.assert_allclose(y, dense[toks], rtol=1e-12, atol=1e-10)
    for c, (toks, act, y) in F.adas_ffn_cubes(x, g, 1e-9, wg, wu, wd).items():
        big = int(np.argmax(np.linalg.norm(x[toks], axis=1)))
        assert act.tolist() == [big]
        f_big = dense[toks[big]] - x[toks[big]]
        np.testing.assert_allclose(y - x[toks], np.broadcast_to(f_big, y.shape), rtol=1e-12, atol=1e-10)


def test_text_tokens_are_dense_regardless_of_p():
    rng = np.random.default_rng(4)
    xt = rng.standard_normal((5, 16))
    wg, wu, wd = rng.standard_normal((24, 16)), rng.standard_normal((24, 16)), rng.standard_normal((16, 24))
    np.testing.assert_allclose(F.adas_ffn_text(xt, wg, wu, wd), xt + _torch_swiglu(xt, wg, wu, wd),
                               rtol=1e-12, atol=1e-10)


def test_tiny_workload_keep_ratio_adapts_to_the_cube():
    wl = workloads.get_ffn("ffn_tiny")
    d = workloads.generate_ffn(wl)
    g = O.Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw)
    sel = F.ffn_select(d["x"], g, wl.p)
    counts = sorted(len(a) for _, a in sel.values())
    # busy cubes (wide magnitude spread) keep fewer tokens than flat ones
    assert counts[0] < counts[-1]
    assert all(1 <= k <= g.S for k in counts)

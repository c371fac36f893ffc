"""Pins for the oracle's attention over the selected cubes plus the own cube (O6).

AdaSpark, papernotes.org, key design 2: each query attends to the Top-p cube
set and always keeps full attention to its own cube.  At p = 1 every
preceding cube is selected, so the result must be dense block-causal
attention, a textbook masked-softmax routine.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import adas_oracle as O
from tests.conftest import GOLDEN


def _setup(wl):
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, perm = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    kbar = O.mean_keys(k_cube, g)
    return data, g, q_cube, k_cube, v_cube, perm, kbar


def _raster(outputs, perm, N, Hq, d):
    out = np.full((N, Hq, d), np.nan)
    for (hq, pos), o in outputs.items():
        out[perm[pos], hq] = o
    return out


def test_attention_golden():
    gold = json.load(open(os.path.join(GOLDEN, "attention_cases.json")))
    for case in gold["cases"]:
        o = O.attend(np.array(case["q"]), np.array(case["keys"]), np.array(case["values"]))
        np.testing.assert_allclose(o, case["out"], rtol=0, atol=1e-13)


GQA_SMALL = workloads.Workload(name="gqa_small", T=4, H=8, W=8, ct=2, ch=4, cw=4,
                               n_q_heads=4, n_kv_heads=2, head_dim=16, dtype="bf16",
                               p=1.0, seed=21)


@pytest.mark.parametrize("wl", [workloads.get("tiny", p=1.0), workloads.get("tiny_b", p=1.0), GQA_SMALL],
                         ids=["tiny", "tiny_b", "gqa_bf16"])
def test_p1_equals_dense_block_causal(wl):
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    sel = O.select_video_rows(q_cube, kbar, g, 1.0)
    for (hq, pos), S in sel.items():
        assert S.tolist() == list(range(pos // g.S))
    got = _raster(O.attention_video_rows(q_cube, k_cube, v_cube, g, sel), perm,
                  g.N, wl.n_q_heads, wl.head_dim)
    ref = O.dense_block_causal(data["q"], data["k"], data["v"], g)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_dense_block_causal_matches_torch_sdpa():
    wl = GQA_SMALL
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    ref = O.dense_block_causal(data["q"], data["k"], data["v"], g)
    q = torch.from_numpy(O.to_f64(data["q"])).permute(1, 0, 2)          # [Hq][N][d]
    k = torch.from_numpy(O.to_f64(data["k"])).permute(1, 0, 2)
    v = torch.from_numpy(O.to_f64(data["v"])).permute(1, 0, 2)
    rep = wl.n_q_heads // wl.n_kv_heads
    k = k.repeat_interleave(rep, dim=0)
    v = v.repeat_interleave(rep, dim=0)
    # cube ids by an independent route: block coordinates of a meshgrid
    f, y, x = np.meshgrid(np.arange(wl.T), np.arange(wl.H), np.arange(wl.W), indexing="ij")
    cid = ((f // wl.ct) * (wl.H // wl.ch) * (wl.W // wl.cw) + (y // wl.ch) * (wl.W // wl.cw)
           + x // wl.cw).reshape(-1)
    mask = torch.from_numpy(cid[None, :] <= cid[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    np.testing.assert_allclose(out.permute(1, 0, 2).numpy(), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("p", [0.3, 0.7])
def test_gather_route_equals_dense_mask_route(p):
    """For the oracle's own Top-p sets, gathering cube tokens gives the same
    output as a dense N x N mask built from those sets."""
    wl = GQA_SMALL.replace(p=p)
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    sel = O.select_video_rows(q_cube, kbar, g, p)
    got = O.attention_video_rows(q_cube, k_cube, v_cube, g, sel)
    kf, vf = O.to_f64(k_cube), O.to_f64(v_cube)
    d = wl.head_dim
    cube_of_pos = np.arange(g.N) // g.S
    for (hq, pos), S in sel.items():
        kv = hq // (wl.n_q_heads // wl.n_kv_heads)
        allowed = np.isin(cube_of_pos, np.append(S, pos // g.S))
        s = kf[kv] @ O.to_f64(q_cube[hq, pos]) / math.sqrt(d)
        s = np.where(allowed, s, -np.inf)
        w = np.exp(s - s.max())
        w /= w.sum()
        np.testing.assert_allclose(got[(hq, pos)], w @ vf[kv], rtol=0, atol=1e-12)


def test_first_cube_rows_are_dense_within_the_cube():
    wl = workloads.get("tiny")
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    sel = O.select_video_rows(q_cube, kbar, g, wl.p, cubes=[0])
    got = O.attention_video_rows(q_cube, k_cube, v_cube, g, sel)
    kf, vf, qf = O.to_f64(k_cube[0, :g.S]), O.to_f64(v_cube[0, :g.S]), O.to_f64(q_cube[0, :g.S])
    s = qf @ kf.T / math.sqrt(wl.head_dim)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    for r in range(g.S):
        np.testing.assert_allclose(got[(0, r)], (w @ vf)[r], rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    wl = GQA_SMALL.replace(p=0.6)
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    sel = O.select_video_rows(q_cube, kbar, g, wl.p)
    got = O.attention_video_rows(q_cube, k_cube, v_cube, g, sel)
    rep = wl.n_q_heads // wl.n_kv_heads
    k_rep, v_rep = np.repeat(k_cube, rep, axis=0), np.repeat(v_cube, rep, axis=0)
    kbar_rep = O.mean_keys(k_rep, g)
    sel_rep = O.select_video_rows(q_cube, kbar_rep, g, wl.p)
    assert all(np.array_equal(sel[k], sel_rep[k]) for k in sel)
    mha = O.attention_video_rows(q_cube, k_rep, v_rep, g, sel_rep)
    for key in got:
        np.testing.assert_array_equal(got[key], mha[key])


def test_explicit_head_map_matches_default():
    wl = GQA_SMALL.replace(p=0.6)
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    hm = np.array([0, 0, 1, 1])
    a = O.select_video_rows(q_cube, kbar, g, wl.p)
    b = O.select_video_rows(q_cube, kbar, g, wl.p, head_map=hm)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    # swapping the map sends heads to the other KV head
    c = O.select_video_rows(q_cube, kbar[::-1].copy(), g, wl.p, head_map=np.array([1, 1, 0, 0]))
    assert all(np.array_equal(a[k], c[k]) for k in a)


def test_within_cube_permutation_only_permutes_outputs():
    """Key design 1/2: selection sees only cube means and attention sees whole
    cubes, so reordering keys inside a cube changes nothing and reordering
    queries inside a cube only reorders the outputs."""
    wl = GQA_SMALL.replace(p=0.6)
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    sel = O.select_video_rows(q_cube, kbar, g, wl.p)
    base = O.attention_video_rows(q_cube, k_cube, v_cube, g, sel)
    rng = np.random.default_rng(9)
    pi = np.concatenate([c * g.S + rng.permutation(g.S) for c in range(g.n_cubes)])
    k2, v2 = k_cube[:, pi], v_cube[:, pi]
    kbar2 = O.mean_keys(k2, g)
    sel2 = O.select_video_rows(q_cube, kbar2, g, wl.p)
    out2 = O.attention_video_rows(q_cube, k2, v2, g, sel2)
    for key in base:
        np.testing.assert_array_equal(sel[key], sel2[key])
        np.testing.assert_allclose(out2[key], base[key], rtol=0, atol=1e-12)
    q2 = q_cube[:, pi]
    sel3 = O.select_video_rows(q2, kbar, g, wl.p)
    out3 = O.attention_video_rows(q2, k_cube, v_cube, g, sel3)
    for hq in range(wl.n_q_heads):
        for pos in range(g.N):
            np.testing.assert_array_equal(out3[(hq, pos)], base[(hq, int(pi[pos]))])


def test_outputs_are_convex_combinations_of_attended_values():
    wl = GQA_SMALL.replace(p=0.5)
    data, g, q_cube, k_cube, v_cube, perm, kbar = _setup(wl)
    sel = O.select_video_rows(q_cube, kbar, g, wl.p)
    got = O.attention_video_rows(q_cube, k_cube, v_cube, g, sel)
    vf = O.to_f64(v_cube)
    for (hq, pos), o in got.items():
        kv = hq // 2
        cubes = sorted(set(sel[(hq, pos)].tolist()) | {pos // g.S})
        vals = np.concatenate([vf[kv, j * g.S:(j + 1) * g.S] for j in cubes])
        assert np.all(o <= vals.max(axis=0) + 1e-12) and np.all(o >= vals.min(axis=0) - 1e-12)


def test_text_rows_p1_equal_dense_over_video_and_causal_text():
    wl = GQA_SMALL.replace(n_text=6, text_kv=True)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    kbar = O.mean_keys(k_cube, g)
    sel = O.select_extra_rows(data["q_text"], kbar, 1.0)
    kf, vf = O.to_f64(data["k"]), O.to_f64(data["v"])
    kt, vt = O.to_f64(data["k_text"]), O.to_f64(data["v_text"])
    for (hq, m), S in sel.items():
        assert S.tolist() == list(range(g.n_cubes))
        o = O.attention_extra_row(data["q_text"], k_cube, v_cube, g, hq, m, S,
                                  data["k_text"], data["v_text"])
        kv = hq // 2
        keys = np.concatenate([kf[:, kv], kt[: m + 1, kv]])
        vals = np.concatenate([vf[:, kv], vt[: m + 1, kv]])
        s = keys @ O.to_f64(data["q_text"][m, hq]) / math.sqrt(wl.head_dim)
        w = np.exp(s - s.max())
        np.testing.assert_allclose(o, (w / w.sum()) @ vals, rtol=0, atol=1e-12)


def test_decode_rows_attend_selected_cubes_only():
    wl = GQA_SMALL.replace(video_queries=False, n_decode=3, p=0.5)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    kbar = O.mean_keys(k_cube, g)
    sel = O.select_extra_rows(data["q_text"], kbar, wl.p)
    for (hq, m), S in sel.items():
        o = O.attention_extra_row(data["q_text"], k_cube, v_cube, g, hq, m, S)
        kv = hq // 2
        keys = np.concatenate([O.to_f64(k_cube[kv, j * g.S:(j + 1) * g.S]) for j in S])
        vals = np.concatenate([O.to_f64(v_cube[kv, j * g.S:(j + 1) * g.S]) for j in S])
        s = keys @ O.to_f64(data["q_text"][m, hq]) / math.sqrt(wl.head_dim)
        w = np.exp(s - s.max())
        np.testing.assert_allclose(o, (w / w.sum()) @ vals, rtol=0, atol=1e-12)

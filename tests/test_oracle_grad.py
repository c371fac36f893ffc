"""Pins of the attention-gradient oracle (oracle/grad_oracle.py) against torch
autograd (an independent implementation of the same derivative), central
finite differences and identities of the softmax derivative."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import workloads
from oracle import adas_oracle as O
from oracle import grad_oracle as G


def _torch_row(q, keys, values, do):
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(keys, requires_grad=True)
    vt = torch.tensor(values, requires_grad=True)
    o = torch.softmax((kt @ qt) / math.sqrt(q.shape[-1]), dim=0) @ vt
    o.backward(torch.tensor(do))
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_row_gradient_matches_torch_autograd():
    rng = np.random.default_rng(0)
    for n, d in ((1, 8), (5, 16), (40, 64)):
        q, k, v, do = (rng.standard_normal(d), rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d)),
                       rng.standard_normal(d))
        o, lse, dq, dk, dv = G.attend_grad(q, k, v, do)
        to, tq, tk, tv = _torch_row(q, k, v, do)
        np.testing.assert_allclose(o, to, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dq, tq, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv, rtol=1e-10, atol=1e-12)
        assert abs(lse - logsumexp(k @ q / math.sqrt(d))) < 1e-12


def test_row_gradient_matches_finite_differences():
    rng = np.random.default_rng(1)
    n, d = 6, 8
    q, k, v, do = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal(d)
    _, _, dq, dk, dv = G.attend_grad(q, k, v, do)
    loss = lambda q_, k_, v_: float(G.attend_grad(q_, k_, v_, do)[0] @ do)
    h = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1, args2 = [q, k, v], [q, k, v]
            args1[which], args2[which] = a1, a2
            num[idx] = (loss(*args1) - loss(*args2)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_softmax_derivative_identities():
    rng = np.random.default_rng(2)
    q, k, v, do = rng.standard_normal(32), rng.standard_normal((50, 32)), rng.standard_normal((50, 32)), rng.standard_normal(32)
    o, _, dq, dk, dv = G.attend_grad(q, k, v, do)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)       # sum_j ds_j = 0
    np.testing.assert_allclose(dv.sum(axis=0), do, rtol=1e-12, atol=1e-12)  # sum_j p_j = 1
    # shifting every key by the same vector leaves p, o and dq unchanged
    _, _, dq2, _, _ = G.attend_grad(q, k + rng.standard_normal(32), v, do)
    np.testing.assert_allclose(dq, dq2, rtol=1e-9, atol=1e-12)


def test_p_one_gradients_equal_dense_block_causal_autograd():
    wl = workloads.get("tiny").replace(name="tiny_grad", n_q_heads=2, n_kv_heads=1)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, _ = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    rng = np.random.default_rng(3)
    dout = rng.standard_normal((g.N, wl.n_q_heads, wl.head_dim))
    sel = {(hq, p): list(range(p // g.S)) for hq in range(wl.n_q_heads) for p in range(g.N)}
    res = G.attention_grads(q_cube, k_cube, v_cube, g, sel, dout)
    # independent route: dense masked attention in raster order, torch autograd
    q = torch.tensor(O.to_f64(data["q"]), requires_grad=True)
    k = torch.tensor(O.to_f64(data["k"]), requires_grad=True)
    v = torch.tensor(O.to_f64(data["v"]), requires_grad=True)
    cube, _ = O.cube_coords(g, np.arange(g.N))
    mask = torch.tensor(cube[None, :] <= cube[:, None])
    outs = []
    for hq in range(wl.n_q_heads):
        s = (q[:, hq] @ k[:, 0].T) / math.sqrt(wl.head_dim)
        s = s.masked_fill(~mask, float("-inf"))
        outs.append(torch.softmax(s, dim=1) @ v[:, 0])
    o = torch.stack(outs, dim=1)
    o.backward(torch.tensor(dout))
    np.testing.assert_allclose(res["dq_raster"], q.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dk_raster"], k.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dv_raster"], v.grad.numpy(), rtol=1e-9, atol=1e-10)


def test_sparse_rows_equal_masked_autograd_and_extra_rows():
    wl = workloads.get("tiny")
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, _ = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    kbar = O.mean_keys(k_cube, g)
    sel = O.select_video_rows(q_cube, kbar, g, 0.5)
    rng = np.random.default_rng(4)
    dout = rng.standard_normal((g.N, 1, wl.head_dim))
    qx = rng.standard_normal((3, 1, wl.head_dim))
    dox = rng.standard_normal((3, 1, wl.head_dim))
    selx = {(0, m): sorted(rng.choice(g.n_cubes, size=3 + m, replace=False).tolist()) for m in range(3)}
    res = G.attention_grads(q_cube, k_cube, v_cube, g, sel, dout, qx, selx, dox)
    # torch: one masked dense softmax per row over the raster keys
    k = torch.tensor(O.to_f64(data["k"])[:, 0], requires_grad=True)
    v = torch.tensor(O.to_f64(data["v"])[:, 0], requires_grad=True)
    cube, _ = O.cube_coords(g, np.arange(g.N))
    qr = torch.tensor(O.to_f64(data["q"])[:, 0], requires_grad=True)
    qxt = torch.tensor(qx[:, 0], requires_grad=True)
    loss = 0
    perm = O.partition(data["q"], g)[1]
    for (hq, p), cubes in sel.items():
        n = int(perm[p])
        allowed = torch.tensor(np.isin(cube, list(cubes) + [p // g.S]))
        s = (k @ qr[n]) / math.sqrt(wl.head_dim)
        o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=0) @ v
        loss = loss + o @ torch.tensor(dout[n, 0])
    for (hq, m), cubes in selx.items():
        allowed = torch.tensor(np.isin(cube, cubes))
        s = (k @ qxt[m]) / math.sqrt(wl.head_dim)
        o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=0) @ v
        loss = loss + o @ torch.tensor(dox[m, 0])
    loss.backward()
    np.testing.assert_allclose(res["dq_raster"][:, 0], qr.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dk_raster"][:, 0], k.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dv_raster"][:, 0], v.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dq_extra"][:, 0], qxt.grad.numpy(), rtol=1e-9, atol=1e-10)


def test_text_rows_with_causal_text_keys_equal_masked_autograd():
    """Text rows of a prefill attend their selected video cubes and the text
    tokens up to themselves; the gradients of the text keys and values collect
    from every later text row (torch autograd over one masked softmax per row)."""
    wl = workloads.get("tiny").replace(name="tiny_text_grad", n_q_heads=2, n_kv_heads=1, n_text=5, text_kv=True)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, _ = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    rng = np.random.default_rng(5)
    nt, Hq, d = wl.n_text, wl.n_q_heads, wl.head_dim
    dox = rng.standard_normal((nt, Hq, d))
    selx = {(hq, m): sorted(rng.choice(g.n_cubes, size=2 + m, replace=False).tolist())
            for hq in range(Hq) for m in range(nt)}
    qx = O.to_f64(data["q_text"])
    res = G.attention_grads(q_cube, k_cube, v_cube, g, {}, np.zeros((g.N, Hq, d)), data["q_text"], selx, dox,
                            k_text=data["k_text"], v_text=data["v_text"])
    k = torch.tensor(O.to_f64(data["k"])[:, 0], requires_grad=True)
    v = torch.tensor(O.to_f64(data["v"])[:, 0], requires_grad=True)
    kt = torch.tensor(O.to_f64(data["k_text"])[:, 0], requires_grad=True)
    vt = torch.tensor(O.to_f64(data["v_text"])[:, 0], requires_grad=True)
    qxt = torch.tensor(qx, requires_grad=True)
    cube, _ = O.cube_coords(g, np.arange(g.N))
    loss = 0
    for (hq, m), cubes in selx.items():
        allowed = torch.tensor(np.concatenate([np.isin(cube, cubes), np.arange(nt) <= m]))
        keys = torch.cat([k, kt])
        vals = torch.cat([v, vt])
        s = (keys @ qxt[m, hq]) / math.sqrt(d)
        o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=0) @ vals
        loss = loss + o @ torch.tensor(dox[m, hq])
    loss.backward()
    np.testing.assert_allclose(res["dq_extra"], qxt.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dk_raster"][:, 0], k.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dv_raster"][:, 0], v.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dk_text"][:, 0], kt.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dv_text"][:, 0], vt.grad.numpy(), rtol=1e-9, atol=1e-10)
    # the last text key is attended by the last row only
    assert np.abs(res["dv_text"][-1, 0]).sum() > 0


def test_head_map_routes_every_gradient_to_its_kv_head():
    """Grouped heads with an explicit, non-monotone head map ([1, 0, 1]: query
    heads 0 and 2 read KV head 1): video rows and text rows with causal text
    keys, against torch autograd over one masked softmax per (head, row) that
    reads the mapped KV head, so dK / dV of each KV head collect exactly the
    rows of its query heads."""
    wl = workloads.get("tiny").replace(name="tiny_head_map_grad", n_q_heads=3, n_kv_heads=2, n_text=3,
                                       text_kv=True)
    hm = [1, 0, 1]
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    q_cube, perm = O.partition(data["q"], g)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    rng = np.random.default_rng(6)
    Hq, d, nt = wl.n_q_heads, wl.head_dim, wl.n_text
    rows = [(hq, int(p)) for hq in range(Hq) for p in rng.choice(g.N, size=12, replace=False)]
    sel = {(hq, p): sorted(rng.choice(max(p // g.S, 1), size=min(2, p // g.S), replace=False).tolist())
           for hq, p in rows}
    selx = {(hq, m): sorted(rng.choice(g.n_cubes, size=2, replace=False).tolist()) for hq in range(Hq)
            for m in range(nt)}
    dout = rng.standard_normal((g.N, Hq, d))
    dox = rng.standard_normal((nt, Hq, d))
    res = G.attention_grads(q_cube, k_cube, v_cube, g, sel, dout, data["q_text"], selx, dox, head_map=hm,
                            k_text=data["k_text"], v_text=data["v_text"])
    k = torch.tensor(O.to_f64(data["k"]), requires_grad=True)          # [N][Hkv][d]
    v = torch.tensor(O.to_f64(data["v"]), requires_grad=True)
    kt = torch.tensor(O.to_f64(data["k_text"]), requires_grad=True)    # [nt][Hkv][d]
    vt = torch.tensor(O.to_f64(data["v_text"]), requires_grad=True)
    qr = torch.tensor(O.to_f64(data["q"]), requires_grad=True)         # [N][Hq][d]
    qxt = torch.tensor(O.to_f64(data["q_text"]), requires_grad=True)   # [nt][Hq][d]
    cube, _ = O.cube_coords(g, np.arange(g.N))
    loss = 0
    for (hq, p), cubes in sel.items():
        n = int(perm[p])
        kv = hm[hq]
        allowed = torch.tensor(np.isin(cube, list(cubes) + [p // g.S]))
        s = (k[:, kv] @ qr[n, hq]) / math.sqrt(d)
        o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=0) @ v[:, kv]
        loss = loss + o @ torch.tensor(dout[n, hq])
    for (hq, m), cubes in selx.items():
        kv = hm[hq]
        allowed = torch.tensor(np.concatenate([np.isin(cube, cubes), np.arange(nt) <= m]))
        s = (torch.cat([k[:, kv], kt[:, kv]]) @ qxt[m, hq]) / math.sqrt(d)
        o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=0) @ torch.cat([v[:, kv], vt[:, kv]])
        loss = loss + o @ torch.tensor(dox[m, hq])
    loss.backward()
    np.testing.assert_allclose(res["dq_raster"], qr.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dq_extra"], qxt.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dk_raster"], k.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dv_raster"], v.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dk_text"], kt.grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(res["dv_text"], vt.grad.numpy(), rtol=1e-9, atol=1e-10)
    # both KV heads receive gradient, and KV head 1 from two query heads
    assert np.abs(res["dv_raster"][:, 0]).sum() > 0 and np.abs(res["dv_raster"][:, 1]).sum() > 0

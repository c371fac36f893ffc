"""GPU parity of the sparse-attention backward (adas_sparse_attn_fwd_lse +
adas_sparse_attn_bwd) against the float64 gradient oracle, through the C ABI.

The oracle differentiates the exact attention over the device's (validated)
selection.  bf16 rounding has unit roundoff u = 2^-8.

dq: the device forms D = do . o from the stored bf16 output o, so
|dD| <= u sum_e |do_e o_e|, and every ds_j of the row moves by -p_j dD; with
keys that share a cube centre, dq = c sum_j ds_j k_j is a small difference of
large terms and that shift is not small against it.  It also rounds ds_j to
bf16 for the MFMA (<= u |ds_j|).  Every element is therefore held to the worst-
case bound, from the oracle's p and ds of the row:
    |dq_dev - dq| <= c u (sum_e |do_e o_e| |sum_j p_j k_j| + sum_j |ds_j| |k_j|)
                     + 2e-3 |dq| + 1e-4 rms(dq)
(the last terms: the log-sum-exp, accurate to 1e-3, scales p uniformly; float32
sums).
dk, dv: per gradient row, e = |g_dev - g_ref| / rms of the reference row over
d.  P and dS enter the MFMA products in bf16 (u each, independent signs:
~u/sqrt(3) = 2.3e-3 rms of a sum, ~1.4e-2 at 6 sigma) and dD moves ds by
p_j dD, which does not cancel across rows (their queries are independent):
max e <= 5e-2, mean e <= 5e-3.  The log-sum-exp is checked to 1e-3 (absolute;
bf16 P summed in float32).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import adas_oracle as O
from oracle import grad_oracle as G
from tests.gpu_harness import bits, log, to_dev

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 5e-2, 5e-3


def _geom(wl, head_map=None):
    from adaptive_cube_sparse_amd import Geometry
    return Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, head_map)


def _bf16_normal(rng, shape):
    return workloads.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _lists(layer, wl, g, video_rows=None):
    """Device selection of every row (or of the video rows listed):
    ({(hq, pos): cubes}, {(hq, m): cubes})."""
    cnt = layer.sel_count.cpu().numpy()
    capv = g.S * g.n_cubes * (g.n_cubes - 1) // 2 if wl.video_queries else 0
    n_extra = wl.n_text + wl.n_decode
    sv, sx = {}, {}
    if video_rows is not None:
        # only the listed rows' entries leave the device
        for hq, p in video_rows:
            c, r = divmod(p, g.S)
            o = hq * capv + g.S * c * (c - 1) // 2 + r * c
            sv[(hq, p)] = layer.sel_idx[o:o + int(cnt[hq, p])].cpu().numpy().tolist()
        return sv, sx
    idx = layer.sel_idx.cpu().numpy()
    for hq in range(wl.n_q_heads):
        if wl.video_queries:
            for p in range(g.N):
                c, r = divmod(p, g.S)
                o = hq * capv + g.S * c * (c - 1) // 2 + r * c
                sv[(hq, p)] = idx[o:o + cnt[hq, p]].tolist()
        for m in range(n_extra):
            o = wl.n_q_heads * capv + (hq * n_extra + m) * g.n_cubes
            k = cnt[hq, (g.N if wl.video_queries else 0) + m]
            sx[(hq, m)] = idx[o:o + k].tolist()
    return sv, sx


def _err(got, ref):
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return np.abs(got - ref) / np.maximum(rms, 1e-30)


def _run_case(wl, p=None, seed=0, video_rows=None, key_cubes=None, head_map=None, key_heads=None,
              dq_rows=None):
    """Forward with log-sum-exp and backward on the device, graded against the
    float64 oracle over the device's selection.  video_rows: only these
    (hq, pos) rows are differentiated by the oracle (all rows by default);
    key_cubes: dK and dV are compared on the keys of these cubes only, which
    must be attended by listed rows alone (e.g. the last cubes when every row
    of them is listed); key_heads: KV heads whose dK and dV are compared
    (all by default); dq_rows: video rows (hq, pos) whose dq is held to its
    bound (all differentiated rows by default); head_map: KV head of each
    query head (default hq // (Hq / Hkv))."""
    from adaptive_cube_sparse_amd import AdasAttentionGrad
    p = wl.p if p is None else p
    n_extra = wl.n_text + wl.n_decode
    n_tk = wl.n_text if wl.text_kv else 0
    log(f"[bwd] {wl.name} grid {wl.T}x{wl.H}x{wl.W} cube ({wl.ct},{wl.ch},{wl.cw}) heads {wl.n_q_heads}/"
        f"{wl.n_kv_heads} d {wl.head_dim} p {p} extra {n_extra} causal text keys {n_tk} head_map {head_map}")
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    dev = "cuda:0"
    rng = np.random.default_rng(seed)
    dout = _bf16_normal(rng, (g.N, wl.n_q_heads, wl.head_dim)) if wl.video_queries else None
    doutx = _bf16_normal(rng, (n_extra, wl.n_q_heads, wl.head_dim)) if n_extra else None
    layer = AdasAttentionGrad(_geom(wl, head_map), p, has_video=wl.video_queries, n_extra=n_extra, device=dev,
                              n_text_kv=n_tk)
    qx = to_dev(data["q_text"], dev) if n_extra else None
    kt = to_dev(data["k_text"], dev) if n_tk else None
    vt = to_dev(data["v_text"], dev) if n_tk else None
    layer.forward(to_dev(data["q"], dev) if wl.video_queries else None, to_dev(data["k"], dev),
                  to_dev(data["v"], dev), qx, k_text=kt, v_text=vt)
    dq, dqx, dk, dv = layer.backward(to_dev(dout, dev) if dout is not None else None,
                                     to_dev(doutx, dev) if doutx is not None else None, qx)
    torch.cuda.synchronize()
    sv, sx = _lists(layer.fwd, wl, g, video_rows)
    q_cube = O.partition(data["q"], g)[0] if wl.video_queries else np.zeros((wl.n_q_heads, g.N, wl.head_dim), np.uint16)
    k_cube, _ = O.partition(data["k"], g)
    v_cube, _ = O.partition(data["v"], g)
    ref = G.attention_grads(q_cube, k_cube, v_cube, g, sv, dout if dout is not None else np.zeros((g.N, wl.n_q_heads, wl.head_dim)),
                            data.get("q_text"), sx, doutx, k_text=data.get("k_text") if n_tk else None,
                            v_text=data.get("v_text") if n_tk else None, head_map=head_map)
    # log-sum-exp
    lse = layer.lse.cpu().numpy()
    lerr = 0.0
    for (hq, p_), v in sv.items():
        lerr = max(lerr, abs(lse[hq, p_] - ref["lse"][("v", hq, p_)]))
    for (hq, m), v in sx.items():
        lerr = max(lerr, abs(lse[hq, (g.N if wl.video_queries else 0) + m] - ref["lse"][("x", hq, m)]))
    dq_np = dq.cpu().numpy() if wl.video_queries else None
    dqx_np = dqx.cpu().numpy() if n_extra else None
    # dq: elementwise worst-case bound
    u = 2.0 ** -8
    cs = 1.0 / np.sqrt(wl.head_dim)
    out_dev = O.to_f64(bits(layer.fwd.out_raster)) if wl.video_queries else None
    outx_dev = O.to_f64(bits(layer.fwd.out_extra)) if n_extra else None
    perm = O.partition(data["k"], g)[1]
    worst = 0.0
    rows = [("v", k) for k in sv if dq_rows is None or k in dq_rows] + [("x", k) for k in sx]
    for kind, (hq, r) in rows:
        kv = head_map[hq] if head_map is not None else hq // (wl.n_q_heads // wl.n_kv_heads)
        if kind == "v":
            cubes = sorted(set(sv[(hq, r)]) | {r // g.S})
            n = int(perm[r])
            qv, dov, od = O.to_f64(q_cube[hq, r]), O.to_f64(dout[n, hq]), out_dev[n, hq]
            want = ref["dq_raster"][n, hq]
        else:
            cubes = sx[(hq, r)]
            qv, dov, od = O.to_f64(data["q_text"][r, hq]), O.to_f64(doutx[r, hq]), outx_dev[r, hq]
            want = ref["dq_extra"][r, hq]
        pos = np.concatenate([np.arange(j * g.S, (j + 1) * g.S) for j in cubes]) if cubes else np.zeros(0, int)
        keys, vals = O.to_f64(k_cube[kv][pos]), O.to_f64(v_cube[kv][pos])
        if kind == "x" and n_tk:  # text row r also attends text tokens 0..r
            keys = np.concatenate([keys, O.to_f64(data["k_text"][:r + 1, kv])])
            vals = np.concatenate([vals, O.to_f64(data["v_text"][:r + 1, kv])])
        pw, ds = G.row_weights(qv, keys, vals, dov)
        bound = cs * u * (np.abs(dov * od).sum() * np.abs(pw @ keys) + np.abs(ds) @ np.abs(keys)) \
            + 2e-3 * np.abs(want) + 1e-4 * np.sqrt(np.mean(want ** 2))
        gotv = dq_np[n, hq] if kind == "v" else dqx_np[r, hq]
        ratio = float((np.abs(gotv - want) / bound).max())
        worst = max(worst, ratio)
    log(f"  dq: largest error / bound {worst:.3f} over {len(rows)} rows")
    assert worst <= 1.0
    errs = {}
    keys = slice(None)
    if key_cubes is not None:
        keys = np.sort(np.concatenate([perm[j * g.S:(j + 1) * g.S] for j in key_cubes]))
    kh = slice(None) if key_heads is None else list(key_heads)
    errs["dk"] = _err(dk.cpu().numpy()[keys][:, kh], ref["dk_raster"][keys][:, kh])
    errs["dv"] = _err(dv.cpu().numpy()[keys][:, kh], ref["dv_raster"][keys][:, kh])
    if n_tk:
        errs["dk_text"] = _err(layer.dk_text.cpu().numpy(), ref["dk_text"])
        errs["dv_text"] = _err(layer.dv_text.cpu().numpy(), ref["dv_text"])
    log("  lse max-abs %.2e; " % lerr + ", ".join(f"{k}: max {e.max():.2e} mean {e.mean():.2e}" for k, e in errs.items()))
    assert lerr <= 1e-3
    for k, e in errs.items():
        assert np.all(np.isfinite(e)), k
        assert e.max() <= TOL_MAX and e.mean() <= TOL_MEAN, k
    return layer


def _small(**kw):
    base = dict(name="bwd_small", T=8, H=8, W=8, ct=4, ch=4, cw=4, n_q_heads=4, n_kv_heads=2, head_dim=128,
                dtype="bf16", p=0.6, seed=4101)
    base.update(kw)
    return workloads.Workload(**base)


def test_bwd_video_rows():
    _run_case(_small())


def test_bwd_dense_p1_and_d64_head_groups_of_three():
    _run_case(_small(name="bwd_p1_d64", n_q_heads=6, n_kv_heads=2, head_dim=64, seed=4102), p=1.0)


@pytest.mark.skip(reason="cubes of 128 tokens (two key blocks per cube) faulted the GPU once; the cause is "
                         "not found yet, so the backward rejects S != 64 (ADAS_ERR_SHAPE) until it is")
def test_bwd_cubes_of_128_two_key_blocks():
    _run_case(_small(name="bwd_s128", T=4, H=16, W=16, ct=2, ch=8, cw=8, seed=4103))


def test_bwd_extra_rows_only():
    _run_case(_small(name="bwd_extra", video_queries=False, n_decode=40, seed=4104), p=0.5)


def test_bwd_text_rows_with_causal_text_keys():
    # a text prefill: 20 text rows attend their selected cubes and the text
    # tokens up to themselves, next to the video rows
    _run_case(_small(name="bwd_text", n_text=20, text_kv=True, seed=4107))


def test_bwd_text_only_prefill_two_text_key_rounds():
    # no video rows; 70 text rows (the text kernels' rounds of 64 keys and
    # rows end in a partial round)
    _run_case(_small(name="bwd_text_only", video_queries=False, n_text=70, text_kv=True, seed=4108), p=0.5)


def test_bwd_uneven_head_groups_with_text_keys():
    # 5 query heads on 2 KV heads mapped [0, 0, 1, 1, 1] (groups of 2 and 3):
    # union tiles and key-block row lists span groups of different sizes, and
    # the text keys' dK / dV sum over a group's heads
    _run_case(_small(name="bwd_head_map", n_q_heads=5, n_kv_heads=2, n_text=12, text_kv=True, seed=4109),
              head_map=[0, 0, 1, 1, 1])


def test_bwd_many_cubes_and_tiles():
    # 64 cubes, 7 query heads per KV head: tiles of 256 rows span head slots,
    # early cubes are attended by hundreds of rows
    _run_case(_small(name="bwd_mid", T=16, H=16, W=16, n_q_heads=7, n_kv_heads=1, seed=4105), p=0.7)


def test_bwd_qwen7b_full_size_sampled():
    # the 7B-shaped layer bench.py --backward times (28/4 heads, 1024 cubes of
    # 64, p = 0.7): every row of the last cube for the 7 query heads of KV
    # head 0 (the last cube is attended by its own rows only, so dK and dV of
    # its keys on KV head 0 are then complete sums) plus 2 rows per head in
    # cubes spread over the layer
    wl = workloads.get("qwen7b_p07")
    g = O.Geometry.of(wl)
    Nc, S = g.n_cubes, g.S
    rng = np.random.default_rng(4110)
    rows = {(hq, p) for hq in range(7) for p in range((Nc - 1) * S, Nc * S)}
    for c in (0, 1, Nc // 4, Nc // 2, 3 * Nc // 4, Nc - 3):
        for hq in range(wl.n_q_heads):
            for r in rng.choice(S, size=2, replace=False):
                rows.add((hq, c * S + int(r)))
    spread = {(hq, p) for hq, p in rows if p < (Nc - 1) * S}
    dq_rows = spread | {(hq, p) for hq, p in rows if p >= (Nc - 1) * S and p % 8 == hq}
    _run_case(wl, video_rows=sorted(rows), key_cubes=[Nc - 1], key_heads=[0], dq_rows=dq_rows)


def test_bwd_qwen3b_full_size_sampled():
    # the 3B-shaped layer bench.py --backward times (16/2 heads, 256 cubes of
    # 64, p = 0.7): every row of the last two cubes (so dK and dV of their keys
    # are complete sums) plus 2 rows per head in cubes spread over the layer
    wl = workloads.get("qwen3b")
    g = O.Geometry.of(wl)
    Nc, S = g.n_cubes, g.S
    rng = np.random.default_rng(4106)
    rows = {(hq, p) for hq in range(wl.n_q_heads) for p in range((Nc - 2) * S, Nc * S)}
    for c in (0, 1, Nc // 4, Nc // 2, 3 * Nc // 4, Nc - 3):
        for hq in range(wl.n_q_heads):
            for r in rng.choice(S, size=2, replace=False):
                rows.add((hq, c * S + int(r)))
    _run_case(wl, video_rows=sorted(rows), key_cubes=[Nc - 2, Nc - 1])

"""GPU checks of the streaming KV cache (adas_cache_append): frames appended
in uneven chunks must leave the cache and the mean keys exactly as the
one-pass partition and mean keys of the same prefix (oracle: bit-exact), and a
decode step over the completed cubes must equal the oracle's selection and
attention over that prefix, and the one-pass path bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from oracle import adas_oracle as O
from tests.gpu_harness import TOL_BF16, bits, log, to_dev, to_vt
from oracle.compare import grade_row

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="stream", T=16, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=8, n_kv_heads=2,
                head_dim=128, dtype="bf16", p=0.7, seed=3101, video_queries=False, n_decode=3)
    base.update(kw)
    return workloads.Workload(**base)


def _check_prefix(cache, data, wl, frames):
    """Cache rows of the appended frames and kbar of the completed cubes."""
    hw = wl.H * wl.W
    g = O.Geometry(frames // wl.ct * wl.ct if frames % wl.ct else frames, wl.H, wl.W, wl.ct, wl.ch, wl.cw)
    kc = bits(cache.k_cache)
    vc = bits(cache.v_cache)
    # whole temporal blocks: compare with the one-pass oracle partition of the prefix
    full = frames // wl.ct * wl.ct
    if full:
        gp = O.Geometry(full, wl.H, wl.W, wl.ct, wl.ch, wl.cw)
        k_cube, _ = O.partition(data["k"][: full * hw], gp)
        v_cube, _ = O.partition(data["v"][: full * hw], gp)
        assert np.array_equal(kc[:, : full * hw], k_cube), "K cache differs"
        assert np.array_equal(vc[:, : gp.n_cubes], to_vt(v_cube, gp.S)), "V cache differs"
        kbar = O.kbar_to_f32(O.mean_keys(k_cube, gp))
        got = cache.kbar.cpu().numpy()[:, : gp.n_cubes]
        assert np.array_equal(got.view(np.uint32), kbar.view(np.uint32)), "kbar differs"
    # the unfinished block: its appended frames are in place (compare through
    # a partition of the next whole block, padded with the frames to come)
    if frames % wl.ct:
        nb = full + wl.ct
        gp = O.Geometry(nb, wl.H, wl.W, wl.ct, wl.ch, wl.cw)
        k_cube, _ = O.partition(data["k"][: nb * hw], gp)
        c0 = full // wl.ct * gp.nH * gp.nW
        hwc = wl.ch * wl.cw
        for c in range(c0, gp.n_cubes):
            rows = slice(c * gp.S, c * gp.S + (frames - full) * hwc)
            assert np.array_equal(kc[:, rows], k_cube[:, rows]), f"partial cube {c} differs"


@pytest.mark.parametrize("chunks", [[1, 2, 1, 4, 3, 5], [4, 4, 4, 4], [7, 9]])
def test_stream_append_matches_one_pass(chunks):
    from adaptive_cube_sparse_amd import Geometry, StreamingCache
    wl = _wl()
    log(f"[stream] chunks {chunks} grid {wl.T}x{wl.H}x{wl.W} cube ({wl.ct},{wl.ch},{wl.cw})")
    data = workloads.generate(wl)
    dev = "cuda:0"
    geom = Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    cache = StreamingCache(geom, wl.p, device=dev)
    hw = wl.H * wl.W
    f = 0
    for n in chunks:
        cache.append(to_dev(data["k"][f * hw:(f + n) * hw], dev), to_dev(data["v"][f * hw:(f + n) * hw], dev))
        f += n
        torch.cuda.synchronize()
        _check_prefix(cache, data, wl, f)
    log(f"  {f} frames appended; cache and mean keys match the one-pass layout after every chunk")


def test_stream_full_decode_cache():
    # the decode workload's whole cache (1024 frames of 16x16, 4 KV heads,
    # 4096 cubes) appended in uneven chunks that cross block boundaries:
    # checked mid-block after the second chunk and whole at the end
    from adaptive_cube_sparse_amd import Geometry, StreamingCache
    wl = workloads.get("decode")
    log(f"[stream] full cache {wl.T}x{wl.H}x{wl.W}, {wl.n_kv_heads} KV heads, chunks 3, 258, 763 frames")
    data = workloads.generate(wl)
    dev = "cuda:0"
    geom = Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    cache = StreamingCache(geom, wl.p, device=dev)
    hw = wl.H * wl.W
    f = 0
    for n in (3, 258, 763):
        cache.append(to_dev(data["k"][f * hw:(f + n) * hw], dev), to_dev(data["v"][f * hw:(f + n) * hw], dev))
        f += n
        torch.cuda.synchronize()
        if f in (261, wl.T):
            _check_prefix(cache, data, wl, f)
            log(f"  {f} frames: cache and mean keys equal the one-pass layout")


def test_stream_decode_over_completed_cubes():
    from adaptive_cube_sparse_amd import AdasAttention, Geometry, StreamingCache
    wl = _wl()
    data = workloads.generate(wl)
    dev = "cuda:0"
    geom = Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    cache = StreamingCache(geom, wl.p, device=dev)
    hw = wl.H * wl.W
    q = to_dev(data["q_text"], dev)
    f = 0
    for n in (3, 6, 2, 5):       # completed frames after each: 0, 8, 8, 16
        cache.append(to_dev(data["k"][f * hw:(f + n) * hw], dev), to_dev(data["v"][f * hw:(f + n) * hw], dev))
        f += n
        full = cache.complete_frames
        if full == 0:
            continue
        out, cnt, idx = cache.decode(q)
        torch.cuda.synchronize()
        # the one-pass path over the completed prefix
        wp = wl.replace(T=full)
        gp = Geometry(full, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
        ref = AdasAttention(gp, torch.bfloat16, wl.p, has_video=False, n_extra=wl.n_decode, device=dev)
        ref.build_kv(to_dev(data["k"][: full * hw], dev), to_dev(data["v"][: full * hw], dev))
        ref.decode_step(q)
        torch.cuda.synchronize()
        assert np.array_equal(cnt.cpu().numpy(), ref.sel_count.cpu().numpy())
        Nc = full // wl.ct * (wl.H // wl.ch) * (wl.W // wl.cw)
        for hq in range(wl.n_q_heads):
            for m in range(wl.n_decode):
                o = (hq * wl.n_decode + m) * Nc
                c = int(cnt[hq, m])
                assert np.array_equal(idx[o:o + c].cpu().numpy(), ref.sel_idx[o:o + c].cpu().numpy())
        assert np.array_equal(bits(out), bits(ref.out_extra)), "streaming decode differs from the one-pass path"
        # and the oracle over the prefix
        og = O.Geometry(full, wl.H, wl.W, wl.ct, wl.ch, wl.cw)
        k_cube, _ = O.partition(data["k"][: full * hw], og)
        v_cube, _ = O.partition(data["v"][: full * hw], og)
        kbar = O.mean_keys(k_cube, og)
        errs, grades = [], []
        rep = wl.n_q_heads // wl.n_kv_heads
        for hq in range(wl.n_q_heads):
            for m in range(wl.n_decode):
                o = (hq * wl.n_decode + m) * Nc
                S = idx[o:o + int(cnt[hq, m])].cpu().numpy()
                P = O.selection_probabilities(O.to_f64(data["q_text"][m, hq]), kbar[hq // rep])
                grades.append(grade_row(P, wl.p, S))
                want = O.attention_extra_row(data["q_text"], k_cube, v_cube, og, hq, m, S)
                errs.append(np.abs(O.to_f64(bits(out)[m, hq]) - want))
        e = np.concatenate(errs)
        log(f"  {full} frames: grades {dict((k, grades.count(k)) for k in set(grades))}, max-abs {e.max():.2e}")
        assert "fail" not in grades
        assert e.max() <= TOL_BF16[0] and e.mean() <= TOL_BF16[1]

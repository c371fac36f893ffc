"""Host logic of bench.py, on the CPU: the work counts behind "value" and the
decode roofline, the gate on committed counter traffic, and the one-GPU rule.

The counts are checked against attended key sets and selected-cube unions
enumerated explicitly from the oracle's selection of small seeded workloads,
not against bench.py's closed forms.
"""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

import bench
import workloads
from oracle import adas_oracle as O

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _selection(wl):
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    k_cube = O.partition(data["k"], g)[0]
    kbar = O.mean_keys(k_cube, g)
    sv = O.select_video_rows(O.partition(data["q"], g)[0], kbar, g, wl.p) if wl.video_queries else {}
    n_extra = wl.n_text + wl.n_decode
    sx = O.select_extra_rows(data["q_text"], kbar, wl.p) if n_extra else {}
    return g, sv, sx


def _fake_layer(wl, g, sv, sx):
    """An object with the device layer's selection outputs, on the CPU."""
    n_extra = wl.n_text + wl.n_decode
    nv = g.N if wl.video_queries else 0
    Hq, Nc = wl.n_q_heads, g.n_cubes
    cnt = np.zeros((Hq, nv + n_extra), np.int32)
    idx = np.full(Hq * n_extra * Nc, -1, np.int32)
    for (hq, pos), s in sv.items():
        cnt[hq, pos] = len(s)
    for (hq, m), s in sx.items():
        cnt[hq, nv + m] = len(s)
        off = (hq * n_extra + m) * Nc
        idx[off:off + len(s)] = s
    geom = types.SimpleNamespace(head_dim=wl.head_dim, n_q_heads=Hq, n_kv_heads=wl.n_kv_heads, n_cubes=Nc, S=g.S)
    return types.SimpleNamespace(sel_count=torch.from_numpy(cnt), sel_idx=torch.from_numpy(idx), geom=geom)


def test_attended_pairs_equal_enumerated_key_sets():
    # video rows (selected cubes and the own cube) and text rows with causal
    # text keys, 2 query heads per KV head
    wl = workloads.get("tiny").replace(name="pairs", n_q_heads=2, n_kv_heads=1, n_text=5, text_kv=True, p=0.6)
    g, sv, sx = _selection(wl)
    want = 0
    for (hq, pos), s in sv.items():
        keys = {(int(j), r) for j in s for r in range(g.S)} | {(pos // g.S, r) for r in range(g.S)}
        want += len(keys)
    for (hq, m), s in sx.items():
        keys = {(int(j), r) for j in s for r in range(g.S)} | {("text", t) for t in range(m + 1)}
        want += len(keys)
    assert bench.attended_pairs(_fake_layer(wl, g, sv, sx), wl) == want


def test_attended_pairs_decode_rows_have_no_own_cube():
    wl = workloads.get("tiny").replace(name="pairs_dec", video_queries=False, n_decode=4, n_q_heads=2, n_kv_heads=1)
    g, sv, sx = _selection(wl)
    want = sum(len(s) * g.S for s in sx.values())
    assert bench.attended_pairs(_fake_layer(wl, g, sv, sx), wl) == want


def test_decode_bytes_count_each_kv_heads_union_once():
    # 4 query heads over 2 KV heads, 3 decode rows: a cube selected by several
    # rows of one KV head is read once for that head
    wl = workloads.get("tiny").replace(name="dec_bytes", video_queries=False, n_decode=3, n_q_heads=4, n_kv_heads=2,
                                       dtype="bf16", p=0.5)
    g, sv, sx = _selection(wl)
    layer = _fake_layer(wl, g, sv, sx)
    rep = wl.n_q_heads // wl.n_kv_heads
    kv_bytes = 0
    for kv in range(wl.n_kv_heads):
        union = set()
        for (hq, m), s in sx.items():
            if hq // rep == kv:
                union |= set(int(j) for j in s)
        kv_bytes += len(union) * g.S * wl.head_dim * 2 * 2  # K and V, bf16
    entries = sum(len(s) for s in sx.values())
    rows = wl.n_q_heads * wl.n_decode
    want = kv_bytes + 2 * rows * wl.head_dim * 2 + 4 * entries + 4 * rows  # + queries, outputs, lists, counts
    assert bench.decode_unique_bytes(layer, wl) == want


def test_counter_traffic_reported_only_for_matching_sources(monkeypatch):
    rec = bench.traffic_entry("hour")
    assert rec is not None and rec > 0  # the committed counters match the committed sources
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.traffic_entry("hour") is None
    assert bench.traffic_entry("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

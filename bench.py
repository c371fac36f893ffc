#!/usr/bin/env python3
"""Throughput of the AdaS-Attn hot path on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic
input already resident in HBM: cube partition of Q, K and V, cube mean keys,
Top-p selection and sparse attention (for the decode workload: selection and
attention of one decode step over a cache built before timing).

The printed JSON line reports:
  value       effective TFLOP/s = 4 * d * (attended (row, key) pairs) / step
              time, counting only the tokens each row attends (selected
              cubes, own cube, causal text);
  roofline    the attention call alone (adas_sparse_attn_fwd: the kernels
              listed under "kernels"): algorithmic FLOPs (or bytes for
              decode) per call / its mean duration, timed with HIP events on
              the launch stream inside the timed region, against the MI355X
              peak; "traffic" is the counter-measured HBM bytes per call when
              profiles/attn_traffic.json matches the current sources;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload.

With an AdaS-FFN workload (--config ffn3b, ffn7b, ffn_hour, ffn_tiny) a step
is instead one AdaS-FFN layer: per-cube token selection, then the FFN of the
active and text tokens plus mean compensation of the skipped ones; "value" is
6 * hidden * inter * (active + text tokens) FLOPs per step time, and the
roofline covers the adas_ffn_fwd call (its two GEMMs and the combine pass).

With --backward (video workloads, cubes of 64 tokens) a step is one
fine-tuning pass of the attention: partition, selection and the forward with
its log-sum-exp, then the backward with the selection held fixed; "value" is
(4 + 10) * d * (attended pairs) FLOPs per step time (forward: QK^T and PV;
backward: S, dP, dV, dK and dQ), and the roofline covers the
adas_sparse_attn_bwd call at 10 * d FLOPs per attended pair.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "AdaS-Attn effective TFLOP/s (selected tokens) and % of MI355X bf16/HBM peak"
DEFAULT_WORKLOAD = "hour"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD,
                    help="workload name (tiny, qwen3b, qwen7b_p05/p07/p09, hour, decode; AdaS-FFN: "
                         "ffn_tiny, ffn3b, ffn7b, ffn_hour)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--topk", type=int, default=0,
                    help="select the K most probable cubes per row instead of Top-p (a timing "
                         "control: fixed budget versus the adaptive one)")
    ap.add_argument("--decode-batch", type=int, default=1,
                    help="decode tokens per step for the decode workload (1 = one step)")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward of the sparse attention (selection held fixed)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the peak probes (MFMA-only loop, HBM read and copy streams)")
    ap.add_argument("--no-flush", action="store_true",
                    help="decode: do not flush the caches between steps")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (for scaling "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


ATTN_SOURCES = ("attn.hip", "attn_union.hip", "attn_decode.hip", "common.h")


def source_hash() -> str:
    """sha256 prefix over the sources of the kernels one adas_sparse_attn_fwd
    call launches (the counters in profiles/ are valid only for these)."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "adaptive_cube_sparse_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def attention_kernels(wl, n_extra: int) -> list:
    """Kernels launched by one adas_sparse_attn_fwd call of this workload (the
    event-timed attention interval covers exactly these)."""
    if wl.dtype != "bf16":
        return [f"adas::k_attn_f32<{wl.head_dim}>"]
    d = wl.head_dim
    ks = []
    if n_extra:
        ks.append("adas::k_extra_bitmap")
    rows_per_kv = (wl.n_q_heads // wl.n_kv_heads) * n_extra
    if not wl.video_queries and rows_per_kv <= 32 and wl.cube_size % 64 == 0:
        ks += [f"adas::k_attn_decode<{d}>", f"adas::k_merge_bf16<{d}, 32>"]
    else:
        ks.append(f"adas::k_attn_union<{d}, {'true' if wl.cube_size % 64 == 0 else 'false'}>")
        if not wl.video_queries:
            ks.append(f"adas::k_merge_bf16<{d}, 256>")
    return ks


FFN_SOURCES = ("ffn.hip", "ffn.h", "common.h")


def source_hash_of(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "adaptive_cube_sparse_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def ffn_traffic_entry(workload: str):
    """HBM bytes of one adas_ffn_fwd call from rocprofv3 counters, if the
    committed measurement is for the current FFN sources."""
    path = os.path.join(ROOT, "profiles", "ffn_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except Exception:
        return None
    if not rec or rec.get("ffn_sources_sha256_16") != source_hash_of(FFN_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def traffic_entry(workload: str):
    """HBM traffic of the attention kernel measured with rocprofv3 counters,
    if the committed measurement is for the current kernel source."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except Exception:
        return None
    if not rec or rec.get("attn_sources_sha256_16") != source_hash():
        return None
    return rec.get("bytes_per_launch")


BWD_SOURCES = ("attn_bwd.hip", "attn_bwd.h", "common.h")
BWD_KERNELS = ["adas::k_bwd_prep<{d}>", "adas::k_bwd_dq<{d}>", "adas::k_bwd_lists", "adas::k_bwd_dkdv<{d}>"]


def bwd_traffic_entry(workload: str):
    """HBM bytes of one adas_sparse_attn_bwd call from rocprofv3 counters, if
    the committed measurement is for the current backward sources."""
    path = os.path.join(ROOT, "profiles", "bwd_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except Exception:
        return None
    if not rec or rec.get("bwd_sources_sha256_16") != source_hash_of(BWD_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def attended_pairs(layer, wl) -> int:
    """Sum over rows of the number of keys each row attends."""
    import torch
    S = wl.cube_size
    cnt = layer.sel_count.to(torch.int64)
    total = 0
    nv = wl.n_tokens if wl.video_queries else 0
    if nv:
        total += int(cnt[:, :nv].sum().item()) * S + nv * wl.n_q_heads * S
    n_extra = wl.n_text + wl.n_decode
    if n_extra:
        total += int(cnt[:, nv:].sum().item()) * S
        if wl.text_kv:
            total += wl.n_q_heads * n_extra * (n_extra + 1) // 2
    return total


def decode_unique_bytes(layer, wl) -> int:
    """Algorithmic HBM bytes of one decode attention launch: K and V of every
    cube selected by at least one row of a KV head (read once), plus queries,
    outputs and the selection lists."""
    import torch
    g = layer.geom
    d = g.head_dim
    cnt = layer.sel_count.cpu().numpy()
    idx_all = layer.sel_idx
    Hq, Nc, S = g.n_q_heads, g.n_cubes, g.S
    rep = Hq // g.n_kv_heads
    n_extra = wl.n_decode
    kv_bytes = 0
    list_entries = 0
    for kv in range(g.n_kv_heads):
        used = torch.zeros(Nc, dtype=torch.bool, device=idx_all.device)
        for hq in range(kv * rep, (kv + 1) * rep):
            for m in range(n_extra):
                off = (hq * n_extra + m) * Nc
                c = int(cnt[hq, m])
                used[idx_all[off: off + c].long()] = True
                list_entries += c
        kv_bytes += int(used.sum().item()) * S * d * 2 * 2
    qo = 2 * n_extra * Hq * d * 2
    return kv_bytes + qo + list_entries * 4 + Hq * n_extra * 4


def stage_rates(wl, n_extra: int, st_ms: dict, roof: dict, probes=None) -> dict:
    """Each step of the path against the MI355X peak that bounds it: the
    key pass (K partitioned, read and written once, plus perm and the float32
    mean keys) and the gather of V and Q (read and written once) against
    HBM; the selection's scoring product (2 d flops per candidate of every
    row) against the bf16 MFMA peak; the attention call as in the roofline.
    For decode workloads the key pass and gather are those of the cache
    build, timed once before the steps."""
    el = 2 if wl.dtype == "bf16" else 4
    d, N, Hq, Hkv = wl.head_dim, wl.n_tokens, wl.n_q_heads, wl.n_kv_heads
    S = wl.cube_size
    Nc = N // S
    q_el = N * Hq * d if wl.video_queries else 0
    kv_el = N * Hkv * d
    out = {}
    if "keys" in st_ms:
        b = 2 * el * kv_el + 4 * N + 4 * Hkv * Nc * d
        out["keys"] = {"ms": st_ms["keys"], "bytes": b, "bound": "hbm",
                       "GB/s": b / (st_ms["keys"] * 1e-3) / 1e9,
                       "frac": b / (st_ms["keys"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if "gather" in st_ms:
        b = 2 * el * (q_el + kv_el)
        out["gather"] = {"ms": st_ms["gather"], "bytes": b, "bound": "hbm",
                         "GB/s": b / (st_ms["gather"] * 1e-3) / 1e9,
                         "frac": b / (st_ms["gather"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    cand = (Hq * S * Nc * (Nc - 1) // 2 if wl.video_queries else 0) + Hq * n_extra * Nc
    f = 2.0 * d * cand
    t = f / (st_ms["select"] * 1e-3) / 1e12
    out["select"] = {"ms": st_ms["select"], "scoring_flops": f, "scoring_TFLOP/s": t,
                     "scoring_frac_of_bf16_peak": t / PEAK_BF16_TFLOPS,
                     "bound": "alu (Top-p search; the scoring product is a small share)"}
    out["attention"] = {"ms": roof["launch_ms"], "bound": roof["bound"], "achieved": roof["achieved"],
                        "unit": roof["unit"], "frac": roof["frac"]}
    if probes:
        for k in ("keys", "gather"):
            if k in out:
                out[k]["frac_of_measured"] = out[k]["GB/s"] / probes["hbm_copy_GB/s"]
        out["select"]["scoring_frac_of_measured"] = t / probes["mfma_bf16_TFLOP/s"]
        ref = probes["mfma_bf16_TFLOP/s"] if roof["unit"] == "TFLOP/s" else probes["hbm_read_GB/s"]
        out["attention"]["frac_of_measured"] = roof["achieved"] / ref
    return out


def decode_step_ms(layer, qe_steps, used, flush, flush_sink, stream, graph: bool) -> float:
    """Mean event-timed duration of one decode step through
    ``AdasAttention.decode_step`` (one adas_decode_step call: selection and
    attention), for the same queries the timed loop used, each preceded by
    the cache flush (outside the events).  graph: the step is captured once
    in a HIP graph and replayed, reading its query from a static buffer that
    each step's token is copied into first (also outside the events)."""
    import torch
    q_static = torch.empty_like(qe_steps[0])
    graph_obj = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            q_static.copy_(qe_steps[0])
            layer.decode_step(q_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph_obj = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_obj):
            layer.decode_step(q_static)
        torch.cuda.synchronize()
    else:
        layer.decode_step(qe_steps[0])  # its workspace is allocated on first use
        torch.cuda.synchronize()
    pairs = []
    for j in used:
        if graph:
            q_static.copy_(qe_steps[j])
        if flush is not None:
            torch.sum(flush, dim=0, dtype=torch.int64, out=flush_sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if graph:
            graph_obj.replay()
        else:
            layer.decode_step(qe_steps[j])
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    del graph_obj
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def stream_append_stage(wl, k, v, layer) -> dict:
    """The same video cache built by the streaming path (StreamingCache.append,
    one temporal block of ct frames per call, mean keys formed as each block
    completes): mean event-timed duration per block, its bytes (K and V read
    and written, the block's mean keys written) and whether the streamed cache
    and mean keys equal the one-pass build bit for bit."""
    import torch
    from adaptive_cube_sparse_amd import StreamingCache
    g = layer.geom
    sc = StreamingCache(g, wl.p, device=k.device)
    fr = g.H * g.W
    pairs = []
    for f0 in range(0, g.T, g.ct):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        sc.append(k[f0 * fr:(f0 + g.ct) * fr], v[f0 * fr:(f0 + g.ct) * fr])
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in pairs[1:]]))  # the first call also warms up
    elem = 2  # bf16
    block = g.ct * fr * g.n_kv_heads * g.head_dim * elem * 2   # K and V of one block
    kbar_bytes = (g.H // g.ch) * (g.W // g.cw) * g.n_kv_heads * g.head_dim * 4
    nbytes = 2 * block + kbar_bytes
    same = (torch.equal(sc.k_cache.view(torch.int16), layer.k_cube.view(torch.int16))
            and torch.equal(sc.v_cache.view(torch.int16), layer.v_cube.view(torch.int16))
            and torch.equal(sc.kbar, layer.kbar))
    del sc
    torch.cuda.empty_cache()
    return {"ms_per_block": ms, "frames_per_block": g.ct, "blocks": len(pairs), "bytes_per_block": nbytes,
            "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "matches_one_pass": bool(same),
            "note": "adas_cache_append of one temporal block per call over the whole video, event-timed"}


def peak_probes() -> dict:
    """Measured ceilings: an MFMA-only register loop (dense bf16), the same
    MFMAs with the union attention's side work per MFMA (LDS operand read,
    exp / pack / row-sum, global->LDS staging, barriers: the ceiling of that
    kernel's instruction mix), and streaming HBM reads / copies of 2 GiB (far
    beyond the 256 MB of on-die caches), each timed with HIP events, best of
    three."""
    import torch
    from adaptive_cube_sparse_amd._lib import (adas_probe_attn_mix, adas_probe_hbm_copy, adas_probe_hbm_read,
                                               adas_probe_mfma)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def best(fn, reps=3):
        out = []
        for _ in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return min(out[1:])

    wgs = 2048
    sink = torch.zeros(wgs, dtype=torch.float32, device=dev)
    fl = [0.0]

    def mf():
        fl[0] = adas_probe_mfma(wgs, 2000, sink)
    t = best(mf)
    mfma = fl[0] / t / 1e12
    mix_src = torch.zeros(4 << 20, dtype=torch.uint8, device=dev)
    msink = torch.zeros(1024, dtype=torch.float32, device=dev)
    mix_rate = {}
    for mix in (False, True):
        def mx():
            fl[0] = adas_probe_attn_mix(1024, 1000, mix, mix_src, msink)
        tm = best(mx)
        mix_rate[mix] = fl[0] / tm / 1e12
    del mix_src
    n = 2 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    isink = torch.zeros(8 * 256, dtype=torch.int32, device=dev)
    t_r = best(lambda: adas_probe_hbm_read(src, isink))
    t_c = best(lambda: adas_probe_hbm_copy(src, dst))
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_TFLOP/s": mfma, "hbm_read_GB/s": n / t_r / 1e9, "hbm_copy_GB/s": 2 * n / t_c / 1e9,
            "mfma_random_operands_TFLOP/s": mix_rate[False], "attn_mix_ceiling_TFLOP/s": mix_rate[True],
            "note": "MFMA-only register loop (2048 workgroups x 4 waves x 4 chains); the union attention's "
                    "instruction mix around the same MFMAs and those MFMAs alone, random-mantissa bf16 operands "
                    "(1024 workgroups x 8 waves); 2 GiB streams; best of 3, HIP events"}


def selection_stats(layer, wl) -> dict:
    """What the pages' Figure 4 plots per layer (cubes selected per query),
    from the device lists: mean and quantiles of the selected count, a
    10-bin histogram of the selected fraction of each row's candidates, and
    per-row entropy is not computed (the lists do not carry P)."""
    import torch
    S = wl.cube_size
    Nc = wl.n_tokens // S
    cnt = layer.sel_count.to(torch.float64)
    nv = wl.n_tokens if wl.video_queries else 0
    fr = []
    if nv:
        cand = (torch.arange(nv, device=cnt.device) // S).to(torch.float64)
        keep = cand > 0
        fr.append((cnt[:, :nv] / cand.clamp_min(1))[:, keep].reshape(-1))
    if cnt.shape[1] > nv:
        fr.append((cnt[:, nv:] / Nc).reshape(-1))
    f = torch.cat(fr)
    hist = torch.histc(f, bins=10, min=0.0, max=1.0).to(torch.int64).tolist()
    c_all = cnt.reshape(-1)
    q = torch.quantile(c_all[: min(c_all.numel(), 1 << 24)], torch.tensor([0.5, 0.9, 0.99], dtype=torch.float64,
                                                                           device=cnt.device)).tolist()
    out = {"rows": int(c_all.numel()), "mean_cubes_per_row": float(c_all.mean().item()),
           "p50_p90_p99_cubes": q, "max_cubes": int(c_all.max().item()),
           "selected_fraction_hist": {"edges": [i / 10 for i in range(11)], "counts": hist},
           "mean_selected_fraction": float(f.mean().item())}
    if nv:
        out["video_mean_selected_fraction"] = float(fr[0].mean().item())
    if cnt.shape[1] > nv:
        out["extra_mean_selected_fraction"] = float(fr[-1].mean().item())
    return out


def grade_sample(layer, wl, sample, topk: int = 0) -> dict:
    """Grade the device's lists of the rows the CPU baseline sampled against
    the oracle (exact / within 1e-5 of p / inside the float32 tie window /
    fail), and count the sampled rows whose oracle sum lies within 1e-5 of p."""
    import torch
    from oracle.compare import TOL_MASS, grade_row, grade_row_topk, logit_error_bound
    g = layer.geom
    S, Nc, Hq = g.S, g.n_cubes, g.n_q_heads
    capv = S * Nc * (Nc - 1) // 2 if wl.video_queries else 0
    nv = g.N if wl.video_queries else 0
    n_extra = wl.n_text + wl.n_decode
    cnt = layer.sel_count.cpu().numpy()
    offs, lens = [], []
    for kind, hq, i, *_ in sample:
        if kind == "v":
            c, r = divmod(i, S)
            offs.append(hq * capv + S * c * (c - 1) // 2 + r * c)
            lens.append(int(cnt[hq, i]))
        else:
            offs.append(Hq * capv + (hq * n_extra + i) * Nc)
            lens.append(int(cnt[hq, nv + i]))
    if not sample:
        return {}
    L = max(max(lens), 1)
    idx = torch.tensor(offs, dtype=torch.int64, device=layer.sel_idx.device)[:, None] + \
        torch.arange(L, device=layer.sel_idx.device)[None, :]
    got = layer.sel_idx[idx.clamp_max(layer.sel_idx.numel() - 1)].cpu().numpy()
    grades = {"exact": 0, "near_threshold": 0, "near_tie": 0, "fail": 0}
    near = 0
    for j, (kind, hq, i, q, kb) in enumerate(sample):
        z = (kb @ q) / np.sqrt(q.shape[0])
        e = np.exp(z - z.max()) if len(z) else z
        P = e / e.sum() if len(z) else z
        Sd = got[j, :lens[j]]
        b = logit_error_bound(q, kb, z)
        gr = grade_row_topk(P, topk, Sd, z, b) if topk else grade_row(P, wl.p, Sd, z, b)
        grades[gr] += 1
        if not topk and len(P) and wl.p < 1.0:
            cum = np.cumsum(np.sort(P)[::-1])
            k = int(np.searchsorted(cum, wl.p, side="left")) + 1
            k = min(k, len(P))
            s_k, s_km1 = cum[k - 1], (cum[k - 2] if k >= 2 else 0.0)
            near += int(abs(s_k - wl.p) <= TOL_MASS or abs(s_km1 - wl.p) <= TOL_MASS)
    return {"rows": len(sample), "grades": grades, "oracle_rows_within_1e-5_of_p": near,
            "note": "device lists of the CPU baseline's sampled rows graded against the oracle"}


def cpu_baseline(wl, data, budget_s: float, topk: int = 0, sample_out=None):
    """Time the CPU oracle on a bounded, seeded sample of the workload's rows:
    selection softmax + Top-p + attention per row (partition and mean keys of
    the whole input are timed too).  BLAS is pinned to one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import adas_oracle as O
    rng = np.random.default_rng(123)
    g = O.Geometry.of(wl)
    flops = 0.0
    rows = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        k_cube, _ = O.partition(data["k"], g)
        v_cube, _ = O.partition(data["v"], g)
        q_cube = O.partition(data["q"], g)[0] if wl.video_queries else None
        kbar = O.mean_keys(k_cube, g)
        t_layout = time.perf_counter() - t0
        t_rows = 0.0
        rep = wl.n_q_heads // wl.n_kv_heads
        while t_rows < budget_s:
            hq = int(rng.integers(wl.n_q_heads))
            t1 = time.perf_counter()
            if wl.video_queries:
                pos = int(rng.integers(g.N))
                c = pos // g.S
                P = O.selection_probabilities(O.to_f64(q_cube[hq, pos]), kbar[hq // rep][:c])
                S_ = O.top_k(P, topk) if topk else O.top_p(P, wl.p)
                O.attention_video_row(q_cube, k_cube, v_cube, g, hq, pos, S_)
                keys = (len(S_) + 1) * g.S
                if sample_out is not None:
                    sample_out.append(("v", hq, pos, O.to_f64(q_cube[hq, pos]), kbar[hq // rep][:c]))
            else:
                m = int(rng.integers(wl.n_decode or wl.n_text))
                P = O.selection_probabilities(O.to_f64(data["q_text"][m, hq]), kbar[hq // rep])
                S_ = O.top_k(P, topk) if topk else O.top_p(P, wl.p)
                O.attention_extra_row(data["q_text"], k_cube, v_cube, g, hq, m, S_)
                keys = len(S_) * g.S
                if sample_out is not None:
                    sample_out.append(("x", hq, m, O.to_f64(data["q_text"][m, hq]), kbar[hq // rep]))
            t_rows += time.perf_counter() - t1
            flops += 4.0 * wl.head_dim * keys
            rows += 1
    value = flops / t_rows / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} random rows of {wl.name} (selection softmax, Top-p and attention "
                      f"per row, float64 NumPy, 1 BLAS thread) in {t_rows:.1f} s; whole-input "
                      f"partition + mean keys took {t_layout:.1f} s and are not in the rate",
            "rows_per_s": rows / t_rows, "layout_s": t_layout,
            "host_threads_available": len(os.sched_getaffinity(0))}


def bwd_cpu_baseline(wl, data, budget_s: float):
    """Time the CPU oracle on random video rows of the workload: selection
    softmax, Top-p, then the row's attention and its gradients (float64 NumPy,
    one BLAS thread)."""
    from threadpoolctl import threadpool_limits
    from oracle import adas_oracle as O
    from oracle import grad_oracle as G
    rng = np.random.default_rng(321)
    g = O.Geometry.of(wl)
    rep = wl.n_q_heads // wl.n_kv_heads
    flops, rows, t = 0.0, 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        k_cube, _ = O.partition(data["k"], g)
        v_cube, _ = O.partition(data["v"], g)
        q_cube = O.partition(data["q"], g)[0]
        kbar = O.mean_keys(k_cube, g)
        t_layout = time.perf_counter() - t0
        while t < budget_s:
            hq, pos = int(rng.integers(wl.n_q_heads)), int(rng.integers(g.N))
            kv, c = hq // rep, pos // g.S
            do = rng.standard_normal(wl.head_dim)
            t1 = time.perf_counter()
            qv = O.to_f64(q_cube[hq, pos])
            sel = O.top_p(O.selection_probabilities(qv, kbar[kv][:c]), wl.p)
            cubes = sorted(set(int(j) for j in sel) | {c})
            idx = np.concatenate([np.arange(j * g.S, (j + 1) * g.S) for j in cubes])
            G.attend_grad(qv, O.to_f64(k_cube[kv][idx]), O.to_f64(v_cube[kv][idx]), do)
            t += time.perf_counter() - t1
            flops += 14.0 * wl.head_dim * len(idx)
            rows += 1
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} random video rows of {wl.name} (selection softmax, Top-p, attention and its "
                      f"gradients per row, float64 NumPy, 1 BLAS thread) in {t:.1f} s; whole-input partition "
                      f"+ mean keys took {t_layout:.1f} s and are not in the rate",
            "host_threads_available": len(os.sched_getaffinity(0))}


def bwd_main(args):
    import torch
    import workloads
    from adaptive_cube_sparse_amd import AdasAttentionGrad, Geometry

    wl = workloads.get(args.config)
    if not wl.video_queries or wl.dtype != "bf16" or wl.cube_size != 64 or wl.n_text or wl.n_decode:
        print(f"--backward needs a bf16 video workload with cubes of 64 tokens and no extra rows "
              f"(got {wl.name})", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    data = workloads.generate(wl)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    geom = Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    layer = AdasAttentionGrad(geom, wl.p, has_video=True, n_extra=0, device=dev)
    q, k, v = up(data["q"]), up(data["k"]), up(data["v"])
    gen = torch.Generator(device=dev).manual_seed(wl.seed + 7)
    dout = torch.randn((wl.n_tokens, wl.n_q_heads, wl.head_dim), generator=gen, device=dev).to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    ev = {"forward": [], "backward": []}

    def step(record):
        def mark():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e
        e0 = mark() if record else None
        layer.forward(q, k, v)
        e1 = mark() if record else None
        layer.backward(dout)
        e2 = mark() if record else None
        if record:
            ev["forward"].append((e0, e1))
            ev["backward"].append((e1, e2))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    k_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in p])) for n, p in ev.items()}
    pairs = attended_pairs(layer.fwd, wl)
    d = wl.head_dim
    value = 14.0 * d * pairs / (ms_step * 1e-3) / 1e12
    bwd_flops = 10.0 * d * pairs
    achieved = bwd_flops / (k_ms["backward"] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": bwd_traffic_entry(wl.name),
            "algorithmic_flops_per_launch": bwd_flops,
            "kernels": [k.format(d=d) for k in BWD_KERNELS], "launch_ms": k_ms["backward"]}
    cpu = None if args.no_cpu_baseline else bwd_cpu_baseline(wl, data, args.cpu_seconds)
    out = {
        "metric": "AdaS-Attn forward + backward effective TFLOP/s (selected tokens, selection held fixed) "
                  "and % of MI355X bf16 peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_bwd", "grid": [wl.T, wl.H, wl.W], "cube_thw": [wl.ct, wl.ch, wl.cw],
                   "heads": [wl.n_q_heads, wl.n_kv_heads], "head_dim": d, "p": wl.p,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": k_ms,
        "attended_pairs": pairs,
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
    }
    print(json.dumps(out), flush=True)


FFN_METRIC = "AdaS-FFN effective TFLOP/s (active + text tokens) and % of MI355X bf16 peak"


def ffn_cpu_baseline(wl, data, budget_s: float):
    """Time the CPU oracle (float64 NumPy, one BLAS thread) on whole cubes of
    the workload, drawn at random until the budget is spent."""
    from threadpoolctl import threadpool_limits
    from oracle import adas_oracle as O
    from oracle import ffn_oracle as F
    rng = np.random.default_rng(123)
    g = O.Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw)
    w64 = (O.to_f64(data["w_gate"]), O.to_f64(data["w_up"]), O.to_f64(data["w_down"]))
    flops, cubes, t = 0.0, 0, 0.0
    with threadpool_limits(limits=1):
        while t < budget_s:
            c = int(rng.integers(g.n_cubes))
            t1 = time.perf_counter()
            (toks, act, _), = F.adas_ffn_cubes(data["x"], g, wl.p, None, None, None, cubes=[c],
                                               weights64=w64).values()
            t += time.perf_counter() - t1
            flops += 6.0 * wl.hidden * wl.inter * len(act)
            cubes += 1
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{cubes} random cubes of {wl.name} (norms, Top-p, SwiGLU FFN of the active "
                      f"tokens, mean compensation; float64 NumPy, 1 BLAS thread) in {t:.1f} s",
            "host_threads_available": len(os.sched_getaffinity(0))}


def ffn_main(args):
    import torch
    import workloads
    from adaptive_cube_sparse_amd import AdasFFN, FfnGeometry

    wl = workloads.get_ffn(args.config)
    dev = torch.device("cuda:0")
    data = workloads.generate_ffn(wl)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    geom = FfnGeometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.hidden, wl.inter)
    layer = AdasFFN(geom, wl.p, up(data["w_gate"]), up(data["w_up"]), up(data["w_down"]),
                    n_text=wl.n_text, device=dev)
    x = up(data["x"])
    xt = up(data["x_text"]) if wl.n_text else None
    stream = torch.cuda.current_stream()
    ev = {"select": [], "ffn": []}

    def step(record):
        def mark():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e
        e0 = mark() if record else None
        layer.select(x)
        e1 = mark() if record else None
        layer.ffn(x, xt)
        e2 = mark() if record else None
        if record:
            ev["select"].append((e0, e1))
            ev["ffn"].append((e1, e2))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    k_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in p])) for n, p in ev.items()}
    m_active = int(layer.act_off[-1].item())
    rows = m_active + wl.n_text
    flops = 6.0 * wl.hidden * wl.inter * rows
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (k_ms["ffn"] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": ffn_traffic_entry(wl.name),
            "algorithmic_flops_per_launch": flops,
            "kernels": ["adas::k_ffn_gemm<true>", "adas::k_ffn_gemm<false>", "adas::k_ffn_combine"],
            "launch_ms": k_ms["ffn"]}
    cpu = None if args.no_cpu_baseline else ffn_cpu_baseline(wl, data, args.cpu_seconds)
    out = {
        "metric": FFN_METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "grid": [wl.T, wl.H, wl.W], "cube_thw": [wl.ct, wl.ch, wl.cw],
                   "hidden": wl.hidden, "inter": wl.inter, "p": wl.p, "text_tokens": wl.n_text,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": k_ms,
        "active_tokens": m_active,
        "keep_ratio": m_active / wl.n_tokens,
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_each_way": n * 4, "launches": 3}))
        return
    import workloads
    if args.config in workloads.FFN_WORKLOADS:
        return ffn_main(args)
    if args.backward:
        return bwd_main(args)
    from adaptive_cube_sparse_amd import AdasAttention, Geometry

    wl = workloads.get(args.config)
    decode = not wl.video_queries
    dev = torch.device("cuda:0")
    probes = None if args.no_probes else peak_probes()
    t_gen = time.perf_counter()
    data = workloads.generate(wl)   # decode: all of the workload's decode queries
    t_gen = time.perf_counter() - t_gen
    n_queries = wl.n_decode
    if decode:
        wl = wl.replace(n_decode=args.decode_batch)

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    geom = Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    n_extra = wl.n_text + wl.n_decode
    n_text_kv = wl.n_text if wl.text_kv else 0
    layer = AdasAttention(geom, dt, wl.p, has_video=wl.video_queries, n_extra=n_extra,
                          n_text_kv=n_text_kv, device=dev, topk=args.topk or None)
    q = up(data["q"]) if wl.video_queries else None
    k, v = up(data["k"]), up(data["v"])
    qe = up(data["q_text"]) if n_extra else None
    qe_all = qe
    if decode:
        # each step decodes new query tokens: step i takes tokens
        # (i * batch .. i * batch + batch) mod the workload's count
        qe_all = up(data["q_text"])
        nb = max(1, n_queries // args.decode_batch)
        qe_steps = [qe_all[(i % nb) * args.decode_batch:(i % nb + 1) * args.decode_batch].contiguous()
                    for i in range(nb)]
        qe = qe_steps[0]
    flush = flush_sink = None
    if decode and not args.no_flush:
        # 512 MiB read between decode steps evicts L2 and the memory-side
        # cache (256 MB) and leaves them clean: a written flush would leave
        # dirty lines whose write-back lands inside the timed step
        flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        flush_sink = torch.zeros((), dtype=torch.int64, device=dev)
    kt = up(data["k_text"]) if n_text_kv else None
    vt = up(data["v_text"]) if n_text_kv else None
    stream = torch.cuda.current_stream()
    from adaptive_cube_sparse_amd import ADAS_LAYOUT_VT, adas_cube_partition, adas_cube_partition_keys

    def mark():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def layout(record):
        """The key pass (K partition + mean keys), then V (and Q): the calls of
        AdasAttention.build_kv / partition_queries, with an event between."""
        g = layer.geom
        e0 = mark() if record else None
        adas_cube_partition_keys(g, k, layer.k_cube, layer.perm, layer.kbar)
        e1 = mark() if record else None
        adas_cube_partition(g, v, layer.v_cube, None, layout=ADAS_LAYOUT_VT)
        if q is not None:
            adas_cube_partition(g, q, layer.q_cube, None)
        e2 = mark() if record else None
        return e0, e1, e2

    ev = {name: [] for name in ("layout", "keys", "gather", "select", "attention")}
    if decode:
        # the cache exists before decoding starts; its build is timed once here
        for _ in range(2):
            lay = layout(True)
        torch.cuda.synchronize()
        ev["keys"].append((lay[0], lay[1]))
        ev["gather"].append((lay[1], lay[2]))

    used_queries = []

    def step(record, i=0):
        e0 = e1 = None
        q_i = qe
        if not decode:
            e0, e1, e2 = layout(record)
        else:
            q_i = qe_steps[i % len(qe_steps)]
            if record:
                used_queries.append(i % len(qe_steps))
            if flush is not None:
                torch.sum(flush, dim=0, dtype=torch.int64, out=flush_sink)
            e2 = mark() if record else None
        layer.select(q_i)
        e3 = mark() if record else None
        layer.attend(q_i, kt, vt)
        e4 = mark() if record else None
        if record:
            if not decode:
                ev["layout"].append((e0, e2))  # partition Q/K/V + mean keys
                ev["keys"].append((e0, e1))
                ev["gather"].append((e1, e2))
            ev["select"].append((e2, e3))
            ev["attention"].append((e3, e4))

    for i in range(args.warmup):
        step(False, i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True, args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    wall_ms_step = ms_step

    def mean_ms(pairs):
        return float(np.mean([a.elapsed_time(b) for a, b in pairs])) if pairs else 0.0

    k_ms = {name: mean_ms(p) for name, p in ev.items() if p and name in ("layout", "select", "attention")}
    st_ms = {name: mean_ms(p) for name, p in ev.items() if p}
    sep_ms = None
    if decode and flush is not None:
        # the cache flush between steps is not part of a decode step: the step
        # time is the event-timed selection + attention of each step
        ms_step = k_ms["select"] + k_ms["attention"]
    if decode and args.decode_batch == 1:
        # the library's decode step is one adas_decode_step call: time it over
        # the same queries (and flushes) and take it as the step
        sep_ms = ms_step
        ms_step = decode_step_ms(layer, qe_steps, used_queries, flush, flush_sink, stream, graph=False)
    if decode:
        # every decode query the timed steps used, counted as often as used
        pairs_q, bytes_q = {}, {}
        for j in sorted(set(used_queries)):
            layer.select(qe_steps[j])
            torch.cuda.synchronize()
            pairs_q[j] = attended_pairs(layer, wl)
            bytes_q[j] = decode_unique_bytes(layer, wl)
        pairs = float(np.mean([pairs_q[j] for j in used_queries]))
        alg_bytes = float(np.mean([bytes_q[j] for j in used_queries]))
    else:
        pairs = attended_pairs(layer, wl)
    flops_step = 4.0 * wl.head_dim * pairs
    value = flops_step / (ms_step * 1e-3) / 1e12
    rows = wl.n_q_heads * ((wl.n_tokens if wl.video_queries else 0) + n_extra)
    attn_ms = k_ms["attention"]
    if decode:
        achieved = alg_bytes / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_entry(wl.name),
                "algorithmic_bytes_per_launch": alg_bytes}
    else:
        achieved = flops_step / (attn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_entry(wl.name),
                "algorithmic_flops_per_launch": flops_step}
    roof["kernels"] = attention_kernels(wl, n_extra)
    roof["launch_ms"] = attn_ms  # one adas_sparse_attn_fwd call: the kernels above
    stages = stage_rates(wl, n_extra, st_ms, roof, probes)
    if decode:
        step_gbs = alg_bytes / (ms_step * 1e-3) / 1e9
        stages["decode_step"] = {"ms": ms_step, "bytes": alg_bytes, "bound": "hbm", "GB/s": step_gbs,
                                 "frac": step_gbs / PEAK_HBM_GBS,
                                 "frac_of_measured": (step_gbs / probes["hbm_read_GB/s"]) if probes else None,
                                 "caches_flushed": flush is not None}
        if args.decode_batch == 1:
            stages["decode_step"]["note"] = ("one adas_decode_step call (selection + attention, the "
                                             "selection writing the bitmaps the attention reads)")
            sep_gbs = alg_bytes / (sep_ms * 1e-3) / 1e9
            stages["decode_step_two_calls"] = {
                "ms": sep_ms, "GB/s": sep_gbs, "frac": sep_gbs / PEAK_HBM_GBS,
                "note": "adas_select_topp then adas_sparse_attn_fwd (its own bitmap launch), the timed loop's "
                        "select + attention events"}
            stages["stream_append"] = stream_append_stage(wl, k, v, layer)
            g_ms = decode_step_ms(layer, qe_steps, used_queries, flush, flush_sink, stream, graph=True)
            g_gbs = alg_bytes / (g_ms * 1e-3) / 1e9
            stages["decode_step_graph"] = {
                "ms": g_ms, "GB/s": g_gbs, "frac": g_gbs / PEAK_HBM_GBS,
                "frac_of_measured": (g_gbs / probes["hbm_read_GB/s"]) if probes else None,
                "note": "the same one-call steps (same query rotation and cache flush) replayed from one "
                        "captured HIP graph; event-timed per replay"}

    sel_stats = selection_stats(layer, wl)
    cpu = None
    check = None
    if not args.no_cpu_baseline:
        sample = []
        cpu = cpu_baseline(wl.replace(n_decode=n_queries) if decode else wl, data, args.cpu_seconds,
                           args.topk, sample)
        if decode:
            # the sampled rows come from every decode query: select with each
            # query block that holds some and grade those rows
            B = args.decode_batch
            check = None
            for b in sorted({i_ // B for (_, _, i_, _, _) in sample}):
                if b >= len(qe_steps):
                    continue
                layer.select(qe_steps[b])
                torch.cuda.synchronize()
                part = grade_sample(layer, wl, [(k_, hq, i_ - b * B, q_, kb_) for (k_, hq, i_, q_, kb_)
                                                in sample if i_ // B == b], args.topk)
                if check is None:
                    check = part
                else:
                    check["rows"] += part["rows"]
                    check["oracle_rows_within_1e-5_of_p"] += part["oracle_rows_within_1e-5_of_p"]
                    for key in check["grades"]:
                        check["grades"][key] += part["grades"][key]
        else:
            check = grade_sample(layer, wl, sample, args.topk)
        # the whole step's work at the sampled rate (rows weighted by their work:
        # the step's attention FLOPs over the oracle's FLOP rate), plus its layout
        cpu["full_step_s_extrapolated"] = flops_step / (cpu["value"] * 1e12) + cpu["layout_s"]
    dens = sel_stats.get("video_mean_selected_fraction", sel_stats["mean_selected_fraction"])
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "grid": [wl.T, wl.H, wl.W],
                   "cube_thw": [wl.ct, wl.ch, wl.cw], "heads": [wl.n_q_heads, wl.n_kv_heads],
                   "head_dim": wl.head_dim, "p": wl.p, "topk": args.topk or None,
                   "extra_queries": n_extra,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": k_ms,
        "stages": stages,
        "measured_peaks": probes,
        "queries_per_s": rows / (ms_step * 1e-3),
        "attended_pairs": pairs,
        "mean_selected_fraction": dens,
        "selection": sel_stats,
        "selection_check": check,
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
    }
    if decode:
        out["wall_ms_per_step"] = wall_ms_step
        out["decode_protocol"] = (f"{len(qe_steps)} distinct query tokens in rotation; "
                                  + ("512 MiB read between steps (outside the step's events)"
                                     if flush is not None else "no cache flush"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

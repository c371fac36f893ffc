"""Shared driver for the GPU parity tests: run the HIP path through the C ABI
binding on seeded inputs and compare it with the CPU oracle.

Bars (from the method's contract):
  * cube partition, perm, mean keys: bit-exact;
  * Top-p sets: exact, except rows graded near_threshold / near_tie by
    ``oracle.compare`` (counted and reported, and bounded here);
  * outputs: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3 against float64;
    f32 max-abs <= 1e-4 (float32 accumulation over at most a few thousand
    keys of O(1) values, with ~1e-6 relative exp/scale error).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import workloads
from oracle import adas_oracle as O
from oracle.compare import grade_row, grade_row_topk, logit_error_bound

TOL_BF16 = (2e-2, 2e-3)   # max-abs, mean-abs
TOL_F32 = (1e-4, 1e-5)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dev):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def geometry(wl, head_map=None):
    from adaptive_cube_sparse_amd import Geometry
    return Geometry(wl.T, wl.H, wl.W, wl.ct, wl.ch, wl.cw, wl.n_q_heads, wl.n_kv_heads,
                    wl.head_dim, head_map)


def run_device(wl, data, p=None, head_map=None, dev="cuda:0", k=None):
    """Whole path on the device (Top-k selection when k is given); returns the
    layer object (tensors stay there)."""
    from adaptive_cube_sparse_amd import AdasAttention
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    n_extra = wl.n_text + wl.n_decode
    n_text_kv = wl.n_text if wl.text_kv else 0
    layer = AdasAttention(geometry(wl, head_map), dt, wl.p if p is None else p,
                          has_video=wl.video_queries, n_extra=n_extra, n_text_kv=n_text_kv,
                          device=dev, topk=k)
    q = to_dev(data["q"], dev) if wl.video_queries else None
    qe = to_dev(data["q_text"], dev) if n_extra else None
    kt = to_dev(data["k_text"], dev) if n_text_kv else None
    vt = to_dev(data["v_text"], dev) if n_text_kv else None
    layer.forward(q, to_dev(data["k"], dev), to_dev(data["v"], dev), qe, kt, vt)
    torch.cuda.synchronize()
    return layer


class Reference:
    """Oracle-side state of one workload."""

    def __init__(self, wl, data, head_map=None):
        self.wl, self.data = wl, data
        self.g = O.Geometry.of(wl)
        self.head_map = None if head_map is None else np.asarray(head_map)
        self.k_cube, self.perm = O.partition(data["k"], self.g)
        self.v_cube, _ = O.partition(data["v"], self.g)
        self.q_cube = O.partition(data["q"], self.g)[0] if wl.video_queries else None
        self.kbar = O.mean_keys(self.k_cube, self.g)
        g = self.g
        self.capv = g.S * g.n_cubes * (g.n_cubes - 1) // 2 if wl.video_queries else 0
        self.n_extra = wl.n_text + wl.n_decode
        self.rows_per_head = (g.N if wl.video_queries else 0) + self.n_extra

    def kv(self, hq):
        if self.head_map is not None:
            return int(self.head_map[hq])
        return hq // (self.wl.n_q_heads // self.wl.n_kv_heads)

    # list offsets (adas.h)
    def video_off(self, hq, pos):
        c, r = divmod(pos, self.g.S)
        return hq * self.capv + self.g.S * c * (c - 1) // 2 + r * c

    def extra_off(self, hq, m):
        return self.wl.n_q_heads * self.capv + (hq * self.n_extra + m) * self.g.n_cubes


def vt_columns(S: int) -> np.ndarray:
    """Column of each cube offset in ADAS_LAYOUT_VT (include/adas.h): bits 2
    and 3 swapped inside complete aligned groups of 16, identity in a trailing
    partial group."""
    r = np.arange(S)
    sw = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1)
    return np.where(r < (S & ~15), sw, r)


def to_vt(x_cube: np.ndarray, S: int) -> np.ndarray:
    """[nh][N][d] token-row cube layout -> [nh][Nc][d][S] ADAS_LAYOUT_VT."""
    nh, N, d = x_cube.shape
    t = x_cube.reshape(nh, N // S, S, d).transpose(0, 1, 3, 2)
    out = np.empty_like(t)
    out[..., vt_columns(S)] = t
    return out


def check_layout(ref: Reference, layer):
    """Partition, perm and mean keys: bit-exact."""
    assert np.array_equal(layer.perm.cpu().numpy(), ref.perm), "perm differs"
    assert np.array_equal(bits(layer.k_cube), ref.k_cube), "k_cube differs"
    assert np.array_equal(bits(layer.v_cube), to_vt(ref.v_cube, ref.g.S)), "v_cube (VT layout) differs"
    if ref.q_cube is not None:
        assert np.array_equal(bits(layer.q_cube), ref.q_cube), "q_cube differs"
    kb = layer.kbar.cpu().numpy()
    want = O.kbar_to_f32(ref.kbar)
    assert np.array_equal(kb.view(np.uint32), want.view(np.uint32)), \
        f"kbar differs in {int((kb != want).sum())} entries"


def fetch_lists(ref: Reference, layer, rows):
    """rows: list of ('v', hq, pos) / ('x', hq, m) -> list of int arrays."""
    counts = layer.sel_count.cpu().numpy()
    offs, lens = [], []
    for kind, hq, i in rows:
        if kind == "v":
            offs.append(ref.video_off(hq, i))
            lens.append(int(counts[hq, i]))
        else:
            offs.append(ref.extra_off(hq, i))
            lens.append(int(counts[hq, (ref.g.N if ref.wl.video_queries else 0) + i]))
    maxlen = max(lens) if lens else 0
    if maxlen == 0:
        return [np.zeros(0, np.int32) for _ in rows]
    idx = torch.tensor(offs, dtype=torch.int64, device=layer.sel_idx.device)[:, None] + \
        torch.arange(maxlen, device=layer.sel_idx.device)[None, :]
    idx = idx.clamp_max(layer.sel_idx.numel() - 1)
    got = layer.sel_idx[idx].cpu().numpy()
    return [got[i, :lens[i]] for i in range(len(rows))]


def selection_probs(ref: Reference, kind, hq, i):
    """(P, z, bound) of a row: float64 probabilities and logits over its
    candidates, and the float32 scoring error bound of each logit."""
    kb = ref.kbar[ref.kv(hq)]
    if kind == "v":
        c = i // ref.g.S
        q = O.to_f64(ref.q_cube[hq, i])
        kb = kb[:c]
    else:
        q = O.to_f64(ref.data["q_text"][i, hq])
    z = O.selection_logits(q, kb)
    return O.softmax(z), z, logit_error_bound(q, kb, z)


# Regression alarm, not a correctness bar (every non-exact row is justified on
# its own by the grader): near-tie rows need a cut gap inside the float32
# scoring error, which is about 1e-6 in a logit on these inputs, so they are
# expected in well under 0.1% of rows; near-threshold rows (within 1e-5 of p)
# in about 0.2%.
ALARM_FRAC = 0.01


def check_rows(ref: Reference, layer, rows, p, k=None):
    """Grade the selection of `rows` (Top-p, or Top-k when k is given) and
    compare their outputs."""
    lists = fetch_lists(ref, layer, rows)
    grades = {"exact": 0, "near_threshold": 0, "near_tie": 0, "fail": 0}
    fails = []
    for (kind, hq, i), S in zip(rows, lists):
        P, z, bnd = selection_probs(ref, kind, hq, i)
        gr = grade_row(P, p, S, z, bnd) if k is None else grade_row_topk(P, k, S, z, bnd)
        grades[gr] += 1
        if gr == "fail" and len(fails) < 5:
            want = O.top_p(P, p) if k is None else O.top_k(P, k)
            fails.append((kind, hq, i, S[:10].tolist(), want[:10].tolist()))
    log(f"  selection grades over {len(rows)} rows: {grades}")
    assert grades["fail"] == 0, f"selection failures: {fails}"
    assert grades["near_threshold"] + grades["near_tie"] <= max(2, ALARM_FRAC * len(rows))
    # outputs, with the oracle attending over the device's (validated) sets
    wl = ref.wl
    out_r = bits(layer.out_raster) if layer.out_raster is not None else None
    out_x = bits(layer.out_extra) if layer.out_extra is not None else None
    errs = []
    for (kind, hq, i), S in zip(rows, lists):
        if kind == "v":
            o = O.attention_video_row(ref.q_cube, ref.k_cube, ref.v_cube, ref.g, hq, i, S,
                                      ref.head_map)
            got = O.to_f64(out_r[ref.perm[i], hq])
        else:
            o = O.attention_extra_row(ref.data["q_text"], ref.k_cube, ref.v_cube, ref.g, hq, i, S,
                                      ref.data.get("k_text") if wl.text_kv else None,
                                      ref.data.get("v_text") if wl.text_kv else None, ref.head_map)
            got = O.to_f64(out_x[i, hq])
        errs.append(np.abs(got - o))
    err = np.concatenate(errs) if errs else np.zeros(1)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_F32
    log(f"  outputs: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (tol {tol})")
    assert np.all(np.isfinite(err))
    assert err.max() <= tol[0] and err.mean() <= tol[1]
    return grades, float(err.max()), float(err.mean())


def all_rows(ref: Reference):
    wl, g = ref.wl, ref.g
    rows = []
    if wl.video_queries:
        rows += [("v", hq, pos) for hq in range(wl.n_q_heads) for pos in range(g.N)]
    rows += [("x", hq, m) for hq in range(wl.n_q_heads) for m in range(ref.n_extra)]
    return rows


def sampled_rows(ref: Reference, seed=0, cubes_per_decile=2, tokens_per_cube=4, extra_tokens=16):
    """Seeded stratified sample: query cubes from every decile of cube index
    (plus the first and last cube), a few tokens of each, every head; plus a
    sample of extra tokens (first and last always included)."""
    wl, g = ref.wl, ref.g
    rng = np.random.default_rng(seed)
    rows = []
    if wl.video_queries:
        nc = g.n_cubes
        cubes = {0, nc - 1}
        for d in range(10):
            lo, hi = d * nc // 10, max(d * nc // 10 + 1, (d + 1) * nc // 10)
            cubes.update(rng.integers(lo, hi, size=cubes_per_decile).tolist())
        for c in sorted(cubes):
            toks = rng.choice(g.S, size=min(tokens_per_cube, g.S), replace=False)
            for hq in range(wl.n_q_heads):
                rows += [("v", hq, c * g.S + int(r)) for r in toks]
    if ref.n_extra:
        ms = {0, ref.n_extra - 1}
        ms.update(rng.integers(0, ref.n_extra, size=min(extra_tokens, ref.n_extra)).tolist())
        for m in sorted(ms):
            rows += [("x", hq, m) for hq in range(wl.n_q_heads)]
    return rows

"""CPU checks of the whole-layer selection bookkeeping (``tests/full_select.py``, Top-p and Top-K):
its per-row counts and signatures must agree with the oracle's per-row sets
(``select_video_rows`` / ``select_extra_rows``) packed at the closed-form list
offsets, and a planted change of one list entry must show up."""
import numpy as np

import workloads
from oracle import adas_oracle as O
from tests.full_select import list_signature_numpy, oracle_signatures
from tests.gpu_harness import Reference as CpuReference


def _packed(ref, p, k=None):
    wl, g = ref.wl, ref.g
    Hq = wl.n_q_heads
    counts = np.zeros((Hq, ref.rows_per_head), np.int32)
    cap = Hq * ref.capv + Hq * ref.n_extra * g.n_cubes
    idx = np.full(cap, -7, np.int32)
    nv = g.N if wl.video_queries else 0
    if wl.video_queries:
        for (hq, pos), s in O.select_video_rows(ref.q_cube, ref.kbar, g, p, k=k).items():
            counts[hq, pos] = len(s)
            off = ref.video_off(hq, pos)
            idx[off:off + len(s)] = s
    if ref.n_extra:
        for (hq, m), s in O.select_extra_rows(ref.data["q_text"], ref.kbar, p, k=k).items():
            counts[hq, nv + m] = len(s)
            off = ref.extra_off(hq, m)
            idx[off:off + len(s)] = s
    return counts, idx


def test_signatures_match_oracle_sets():
    wl = workloads.Workload(name="fs", T=8, H=8, W=8, ct=2, ch=4, cw=4, n_q_heads=3, n_kv_heads=1,
                            head_dim=64, dtype="bf16", p=0.7, seed=61, n_decode=5)
    data = workloads.generate(wl)
    ref = CpuReference(wl, data)
    counts, idx = _packed(ref, wl.p)
    oc, osig, near = oracle_signatures(ref, wl.p, workers=2)
    assert np.array_equal(oc, counts)
    sig = list_signature_numpy(counts, idx, ref)
    assert np.array_equal(sig, osig)
    # a planted change of one selected cube id changes that row's signature only
    off = ref.video_off(1, 5 * ref.g.S + 3)
    assert counts[1, 5 * ref.g.S + 3] >= 1
    idx2 = idx.copy()
    idx2[off] = (idx2[off] + 1) % 5
    sig2 = list_signature_numpy(counts, idx2, ref)
    diff = np.argwhere(sig2 != osig)
    assert diff.tolist() == [[1, 5 * ref.g.S + 3]]


def test_topk_signatures_match_oracle_sets():
    # k = 4 below and above the candidate counts of the early cubes (rows of
    # cube c have c candidates and keep all of them while c <= k)
    wl = workloads.Workload(name="fsk", T=8, H=8, W=8, ct=2, ch=4, cw=4, n_q_heads=2, n_kv_heads=1,
                            head_dim=64, dtype="bf16", p=0.7, seed=62, n_decode=3)
    data = workloads.generate(wl)
    ref = CpuReference(wl, data)
    counts, idx = _packed(ref, wl.p, k=4)
    oc, osig, near = oracle_signatures(ref, wl.p, workers=2, k=4)
    assert np.array_equal(oc, counts) and not near.any()
    assert np.array_equal(list_signature_numpy(counts, idx, ref), osig)
    nv = ref.g.N
    assert counts[0, 2 * ref.g.S] == 2 and counts[0, 9 * ref.g.S] == 4 and np.all(counts[:, nv:] == 4)

"""CPU checks of the whole-layer output bookkeeping (``tests/full_outputs.py``):
outputs the oracle itself computed over the oracle's own sets, packed at the
closed-form list offsets and rounded to bf16, must pass within the rounding;
a planted change of one output row, or of one list entry, must show up."""
import numpy as np

import workloads
from oracle import adas_oracle as O
from tests.full_outputs import full_outputs
from tests.gpu_harness import Reference as CpuReference

WL = workloads.Workload(name="fo", T=8, H=8, W=8, ct=2, ch=4, cw=4, n_q_heads=3, n_kv_heads=1,
                        head_dim=64, dtype="bf16", p=0.7, seed=62, n_text=4, text_kv=True)


def _device_like(ref):
    """(counts, packed lists, out_raster bits, out_extra bits) from the oracle."""
    wl, g = ref.wl, ref.g
    Hq = wl.n_q_heads
    counts = np.zeros((Hq, ref.rows_per_head), np.int32)
    idx = np.full(Hq * ref.capv + Hq * ref.n_extra * g.n_cubes, -7, np.int32)
    out_r = np.zeros((g.N, Hq, wl.head_dim), np.float32)
    out_x = np.zeros((ref.n_extra, Hq, wl.head_dim), np.float32)
    for (hq, pos), s in O.select_video_rows(ref.q_cube, ref.kbar, g, wl.p).items():
        counts[hq, pos] = len(s)
        idx[ref.video_off(hq, pos):ref.video_off(hq, pos) + len(s)] = s
        out_r[ref.perm[pos], hq] = O.attention_video_row(ref.q_cube, ref.k_cube, ref.v_cube, g, hq, pos, s)
    for (hq, m), s in O.select_extra_rows(ref.data["q_text"], ref.kbar, wl.p).items():
        counts[hq, g.N + m] = len(s)
        idx[ref.extra_off(hq, m):ref.extra_off(hq, m) + len(s)] = s
        out_x[m, hq] = O.attention_extra_row(ref.data["q_text"], ref.k_cube, ref.v_cube, g, hq, m, s,
                                             ref.data["k_text"], ref.data["v_text"])
    return counts, idx, workloads.f32_to_bf16_bits(out_r), workloads.f32_to_bf16_bits(out_x)


def test_oracle_outputs_pass_and_planted_changes_fail():
    data = workloads.generate(WL)
    ref = CpuReference(WL, data)
    counts, idx, out_r, out_x = _device_like(ref)
    worst, mean, rows = full_outputs(WL, counts, idx, out_r, out_x, ref.perm, chunk_rows=64, workers=2)
    assert rows == WL.n_q_heads * (ref.g.N + WL.n_text)
    assert worst <= 1e-2 and mean <= 2e-3          # bf16 rounding of O(1) outputs
    # one output row off by 0.1 in one element
    bad = out_r.copy()
    v = O.to_f64(bad[ref.perm[40], 2])
    v[7] += 0.1
    bad[ref.perm[40], 2] = workloads.f32_to_bf16_bits(v.astype(np.float32))
    w2, _, _ = full_outputs(WL, counts, idx, bad, out_x, ref.perm, chunk_rows=64, workers=2)
    assert w2 >= 0.09
    # one list entry moved to another (unselected) cube: the oracle then
    # attends a different key set for that row only
    pos = 7 * ref.g.S + 5
    off = ref.video_off(1, pos)
    s = idx[off:off + counts[1, pos]]
    free = sorted(set(range(7)) - set(s.tolist()))
    assert len(s) >= 1 and free
    idx2 = idx.copy()
    idx2[off:off + len(s)] = sorted(set(s.tolist()[1:]) | {free[0]})
    w3, _, _ = full_outputs(WL, counts, idx2, out_r, out_x, ref.perm, chunk_rows=64, workers=2)
    assert w3 > 2e-2
    # a subset of cube positions checks exactly those video rows (and every extra row)
    w4, _, rows4 = full_outputs(WL, counts, idx, bad, out_x, ref.perm, chunk_rows=64, workers=2,
                                positions=[0, 1, 63, 41])
    assert rows4 == WL.n_q_heads * (4 + WL.n_text) and w4 <= 1e-2
    w5, _, _ = full_outputs(WL, counts, idx, bad, out_x, ref.perm, chunk_rows=64, workers=2, positions=[40])
    assert w5 >= 0.09

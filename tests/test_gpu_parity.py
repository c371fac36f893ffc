"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases run every row and span several row tiles with ragged tails;
full-size configurations are checked on seeded stratified row samples.
"""
import numpy as np
import pytest

import workloads
from oracle import adas_oracle as O
from tests.gpu_harness import (Reference, all_rows, check_layout, check_rows, log, run_device,
                               sampled_rows, bits)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _case(wl, p=None, head_map=None, rows="all", k=None, **kw):
    log(f"case {wl.name}: grid {wl.T}x{wl.H}x{wl.W} cube t{wl.ct}h{wl.ch}w{wl.cw} "
        f"heads {wl.n_q_heads}/{wl.n_kv_heads} d {wl.head_dim} {wl.dtype} p {p or wl.p} "
        f"top-k {k} extra {wl.n_text + wl.n_decode} head_map {head_map}")
    data = workloads.generate(wl)
    layer = run_device(wl, data, p=p, head_map=head_map, k=k)
    ref = Reference(wl, data, head_map)
    check_layout(ref, layer)
    rws = all_rows(ref) if rows == "all" else sampled_rows(ref, **kw)
    check_rows(ref, layer, rws, wl.p if p is None else p, k=k)
    return ref, layer


# --- small cases: every row ------------------------------------------------------
SMALL = workloads.Workload(name="small", T=8, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=6,
                           n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=31)


@pytest.mark.parametrize("name", ["tiny", "tiny_b"])
def test_tiny_f32(name):
    _case(workloads.get(name))


@pytest.mark.parametrize("p", [0.05, 0.7, 0.95])
def test_small_bf16(p):
    # 3 heads per KV group x 64 tokens = 192 rows per query cube: 256-row tiles
    # span two query cubes
    _case(SMALL, p=p)


def test_small_bf16_p1_is_dense_block_causal():
    ref, layer = _case(SMALL, p=1.0)
    dense = O.dense_block_causal(ref.data["q"], ref.data["k"], ref.data["v"], ref.g)
    got = O.to_f64(bits(layer.out_raster))
    err = np.abs(got - dense)
    log(f"  p=1 vs dense block-causal: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_small_bf16_head_map_d64():
    wl = SMALL.replace(name="small_d64", head_dim=64, n_q_heads=5, seed=32)
    _case(wl, head_map=[1, 0, 1, 1, 0])


@pytest.mark.parametrize("shape", ["s64_one_head_per_kv", "s128_one_head_per_kv"])
def test_tiles_span_several_query_cubes(shape):
    # one query head per KV head: 64 rows per query cube (a 256-row tile spans
    # four cubes) or 128 rows with two key blocks per cube (two cubes per tile)
    if shape == "s64_one_head_per_kv":
        wl = workloads.Workload(name="span4", T=8, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=2,
                                n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=41)
    else:
        wl = workloads.Workload(name="span2_s128", T=8, H=16, W=16, ct=2, ch=8, cw=8, n_q_heads=3,
                                n_kv_heads=3, head_dim=128, dtype="bf16", p=0.6, seed=42)
    _case(wl)


def test_cubes_of_256_tokens():
    # the training cube of the listing's Table 5, 8x8x4 (h x w x t): four key
    # blocks per cube, 7 query heads per KV head (1792 rows per query cube,
    # so tiles span cube boundaries mid-head), plus text rows
    wl = workloads.Workload(name="cube256", T=16, H=16, W=16, ct=4, ch=8, cw=8, n_q_heads=7,
                            n_kv_heads=1, head_dim=128, dtype="bf16", p=0.8, seed=46,
                            n_text=20, text_kv=True)
    _case(wl)


def test_text_rows_causal_s128():
    # cube 8x8x2 = 128 tokens (two key blocks per cube) + 70 causal text tokens
    wl = workloads.Workload(name="text", T=8, H=16, W=16, ct=2, ch=8, cw=8, n_q_heads=4,
                            n_kv_heads=1, head_dim=128, dtype="bf16", p=0.9, seed=33,
                            n_text=70, text_kv=True)
    _case(wl)


def test_decode_rows_split():
    # extra rows only: the attention splits cubes into chunks and merges them
    wl = workloads.Workload(name="decode_small", T=64, H=16, W=16, ct=4, ch=4, cw=4,
                            n_q_heads=4, n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7,
                            seed=34, video_queries=False, n_decode=5)
    _case(wl)


def test_decode_mode_32_rows_uneven_groups_s128():
    # at most 32 extra rows per KV head run in the per-wave decode kernel: here
    # exactly 32 (4 heads x 8 tokens) on KV head 0 and 8 on KV head 1, with
    # 128-token cubes (two key blocks per cube)
    wl = workloads.Workload(name="decode_32", T=32, H=16, W=16, ct=2, ch=8, cw=8,
                            n_q_heads=5, n_kv_heads=2, head_dim=128, dtype="bf16", p=0.8,
                            seed=36, video_queries=False, n_decode=8)
    _case(wl, head_map=[0, 0, 1, 0, 0])


@pytest.mark.parametrize("p", [0.5, 1.0])
def test_decode_split_selection_2048_cubes(p):
    # few extra rows over more than 1024 cubes take the split selection path
    # (logits in the workspace, one workgroup per row)
    wl = workloads.Workload(name="decode_2048", T=512, H=16, W=16, ct=4, ch=4, cw=4,
                            n_q_heads=5, n_kv_heads=2, head_dim=128, dtype="bf16", p=p,
                            seed=37, video_queries=False, n_decode=3)
    _case(wl, head_map=[0, 0, 1, 1, 1])


def test_many_cubes_small_cube():
    # Nc = 1152 > 1024 candidates (wide selection path), S = 16 (partial key blocks)
    wl = workloads.Workload(name="many_cubes", T=72, H=16, W=16, ct=1, ch=4, cw=4,
                            n_q_heads=2, n_kv_heads=1, head_dim=128, dtype="bf16", p=0.5,
                            seed=35)
    _case(wl, rows="sample", cubes_per_decile=3, tokens_per_cube=8)


def test_extra_rows_with_video_bands_in_one_launch():
    # Nc = 320: the extra rows' 320 candidates and the video rows of cubes
    # 256..319 share the 6-slot band, and the 4-, 2- and 1-slot bands of the
    # earlier cubes run in the same selection launch at their own offsets
    wl = workloads.Workload(name="bands_extra", T=20, H=16, W=16, ct=1, ch=4, cw=4,
                            n_q_heads=4, n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7,
                            seed=41, n_decode=6)
    _case(wl, rows="sample", cubes_per_decile=3, tokens_per_cube=8)


def test_three_block_passes():
    # 3 cubes of 64 tokens, 4 query heads on one KV head: a tile is one query
    # cube (256 rows), so the tile of cube 2 walks exactly three key blocks
    # (own cube 2 plus cubes 1 and 0 whenever a row selects them), the case
    # where the first wait of the four-buffer pipeline has only one block
    # still loading behind the pair it computes
    wl = workloads.Workload(name="three_blocks", T=12, H=4, W=4, ct=4, ch=4, cw=4, n_q_heads=4,
                            n_kv_heads=1, head_dim=128, dtype="bf16", p=0.95, seed=43)
    _case(wl)
    wl = wl.replace(name="three_blocks_d64", head_dim=64, p=0.9, seed=44)
    _case(wl)


def test_text_prefill_without_video_rows():
    # a few text queries with causal text keys and no video rows: at most 32
    # rows per KV head, which is the decode kernel's size, but the decode
    # kernel reads no text keys, so these rows must take the union tiles
    wl = workloads.Workload(name="text_only", T=16, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=4,
                            n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=45,
                            video_queries=False, n_text=6, text_kv=True)
    _case(wl)


def test_max_query_heads_with_text_rows():
    # the largest head count the library takes (ADAS_MAX_HEADS = 128 query
    # heads) over 2 KV heads: 64 query heads per group, so each query cube's
    # rows of a group fill 8 union tiles, and 5 text rows per head give 320
    # extra rows per group (a full extra-row tile and a partial one)
    wl = workloads.Workload(name="max_heads", T=4, H=8, W=8, ct=2, ch=4, cw=4, n_q_heads=128,
                            n_kv_heads=2, head_dim=64, dtype="bf16", p=0.7, seed=46,
                            n_text=5, text_kv=True)
    _case(wl)


def test_single_cube_layer():
    # one cube of 256 tokens (Nc = 1): no video row has a candidate, so every
    # video row attends its own cube only and its list is empty; each text row
    # has the one cube as its only candidate (P = 1), so it selects it
    wl = workloads.Workload(name="one_cube", T=4, H=8, W=8, ct=4, ch=8, cw=8, n_q_heads=4,
                            n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=47,
                            n_text=3, text_kv=True)
    ref, layer = _case(wl)
    cnt = layer.sel_count.cpu().numpy()
    assert (cnt[:, :ref.g.N] == 0).all() and (cnt[:, ref.g.N:] == 1).all()


def test_deterministic():
    data = workloads.generate(SMALL)
    a = run_device(SMALL, data)
    b = run_device(SMALL, data)
    assert torch.equal(a.sel_count, b.sel_count)
    assert torch.equal(a.out_raster.view(torch.int16), b.out_raster.view(torch.int16))


# --- Top-K selection (the listing's Table 4 alternative) -------------------------------
@pytest.mark.parametrize("k", [1, 5, 40])
def test_small_bf16_topk(k):
    # SMALL has 32 cubes: k = 40 keeps every candidate of every row
    _case(SMALL, k=k)


def test_tiny_f32_topk():
    _case(workloads.get("tiny"), k=3)


def test_topk_text_rows_and_split_decode():
    wl = workloads.Workload(name="text_topk", T=8, H=16, W=16, ct=2, ch=8, cw=8, n_q_heads=4,
                            n_kv_heads=1, head_dim=128, dtype="bf16", p=0.9, seed=38,
                            n_text=40, text_kv=True)
    _case(wl, k=3)
    wl = workloads.Workload(name="decode_2048_topk", T=512, H=16, W=16, ct=4, ch=4, cw=4,
                            n_q_heads=5, n_kv_heads=2, head_dim=128, dtype="bf16", p=0.5,
                            seed=39, video_queries=False, n_decode=3)
    _case(wl, head_map=[0, 0, 1, 1, 1], k=300)


# --- full-size configurations: sampled rows ------------------------------------------
@pytest.mark.parametrize("name", ["qwen3b", "qwen7b_p05", "qwen7b_p07", "qwen7b_p09", "hour", "decode"])
def test_full_config_sampled(name):
    _case(workloads.get(name), rows="sample", tokens_per_cube=2, extra_tokens=8)


def test_decode_mode_four_cubes_one_chunk():
    # a decode over a cache of 4 cubes runs the decode kernel as a single
    # chunk: its partial rows still need (and now get) workspace
    wl = workloads.Workload(name="decode_4cubes", T=4, H=8, W=8, ct=4, ch=4, cw=4, n_q_heads=4,
                            n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=39,
                            video_queries=False, n_decode=2)
    _case(wl)


def test_decode_single_step():
    """One decode step (1 query token x 28 heads) over the full decode cache."""
    wl = workloads.get("decode").replace(n_decode=1, name="decode_step")
    _case(wl)


# --- one-call decode step (selection + attention) --------------------------------------
DECODE_STEP_CASES = {
    # 4096 cubes, one query x 28 heads: split selection writes the bitmaps the decode kernel reads
    "cache_4096_one_query": (workloads.get("decode").replace(n_decode=1), None, None),
    # 2048 cubes, 3 queries, uneven head groups: the decode kernel with 9 rows per KV head
    "cache_2048_head_map": (workloads.Workload(name="ds_2048", T=512, H=16, W=16, ct=4, ch=4, cw=4,
                                               n_q_heads=5, n_kv_heads=2, head_dim=128, dtype="bf16",
                                               p=0.6, seed=71, video_queries=False, n_decode=3),
                            [0, 0, 1, 1, 1], None),
    # p = 1: every cube, the bitmaps written by the all-selected branch
    "cache_2048_p1": (workloads.Workload(name="ds_p1", T=512, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=4,
                                         n_kv_heads=2, head_dim=64, dtype="bf16", p=1.0, seed=72,
                                         video_queries=False, n_decode=2), None, None),
    # 56 rows per KV head: split selection, but union tiles read the bitmaps
    "cache_2048_union_tiles": (workloads.Workload(name="ds_union", T=512, H=16, W=16, ct=4, ch=4, cw=4,
                                                  n_q_heads=7, n_kv_heads=1, head_dim=128, dtype="bf16",
                                                  p=0.7, seed=73, video_queries=False, n_decode=8),
                               None, None),
    # 256 cubes: the band selection, the attention builds its own bitmaps
    "cache_256_band_selection": (workloads.Workload(name="ds_band", T=64, H=16, W=16, ct=4, ch=4, cw=4,
                                                    n_q_heads=4, n_kv_heads=2, head_dim=128, dtype="bf16",
                                                    p=0.7, seed=74, video_queries=False, n_decode=2),
                                 None, None),
}


@pytest.mark.parametrize("case", sorted(DECODE_STEP_CASES))
def test_decode_step_call_equals_select_then_attend(case):
    from adaptive_cube_sparse_amd import AdasAttention
    from tests.gpu_harness import geometry, to_dev
    wl, head_map, _ = DECODE_STEP_CASES[case]
    log(f"case {case}: adas_decode_step against adas_select_topp + adas_sparse_attn_fwd "
        f"({wl.n_q_heads}/{wl.n_kv_heads} heads, {wl.T}x{wl.H}x{wl.W}, {wl.n_decode} queries, p {wl.p})")
    data = workloads.generate(wl)
    dev = torch.device("cuda:0")
    layer = AdasAttention(geometry(wl, head_map), torch.bfloat16, wl.p, has_video=False,
                          n_extra=wl.n_decode, device=dev)
    layer.build_kv(to_dev(data["k"], dev), to_dev(data["v"], dev))
    q = to_dev(data["q_text"], dev)
    layer.select(q)
    layer.attend(q)
    torch.cuda.synchronize()
    want = (layer.sel_count.clone(), layer.sel_idx.clone(), layer.out_extra.clone())
    layer.sel_idx.fill_(-5)
    layer.out_extra.zero_()
    layer.decode_step(q)
    torch.cuda.synchronize()
    assert torch.equal(layer.sel_count, want[0])
    cnt = want[0].cpu().numpy()
    got_idx, want_idx = layer.sel_idx.cpu().numpy(), want[1].cpu().numpy()
    Nc = wl.T * wl.H * wl.W // (wl.ct * wl.ch * wl.cw)
    for hq in range(wl.n_q_heads):
        for m in range(wl.n_decode):
            o = (hq * wl.n_decode + m) * Nc
            assert np.array_equal(got_idx[o:o + cnt[hq, m]], want_idx[o:o + cnt[hq, m]]), (hq, m)
    assert torch.equal(layer.out_extra.view(torch.int16), want[2].view(torch.int16))
    # and the rows against the oracle
    ref = Reference(wl, data, head_map)
    check_rows(ref, layer, all_rows(ref), wl.p)

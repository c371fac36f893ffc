"""The allocation-free attention entry point (adas_sparse_attn_fwd_noalloc)
against adas_sparse_attn_fwd with a caller workspace, through the C ABI: both
run the same kernels, so outputs must be bit-identical.  Two calls in a row
on the one per-GPU scratch array, the second on a smaller input, so stale
contents of a larger call must not leak into a smaller one."""
import pytest
import torch

import workloads
from tests.gpu_harness import log, run_device, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _noalloc_matches(wl):
    from adaptive_cube_sparse_amd import adas_sparse_attn_fwd_noalloc
    log(f"case {wl.name}: grid {wl.T}x{wl.H}x{wl.W} heads {wl.n_q_heads}/{wl.n_kv_heads} "
        f"extra {wl.n_text + wl.n_decode} text_kv {wl.text_kv} video {wl.video_queries}")
    data = workloads.generate(wl)
    layer = run_device(wl, data)               # the whole path, attention with a workspace
    assert layer.ws is not None and layer.ws.numel() > 0   # the case does use scratch
    want_r = layer.out_raster.clone() if layer.out_raster is not None else None
    want_x = layer.out_extra.clone()
    if layer.out_raster is not None:
        layer.out_raster.fill_(0)
    layer.out_extra.fill_(0)
    dev = layer.out_extra.device
    kt = vt = None
    if wl.text_kv:
        kt, vt = to_dev(data["k_text"], dev), to_dev(data["v_text"], dev)
    qx = to_dev(data["q_text"], dev)
    adas_sparse_attn_fwd_noalloc(layer.geom, layer.q_cube if wl.video_queries else None, layer.k_cube,
                                 layer.v_cube, qx, kt, vt, layer.sel_count, layer.sel_idx, layer.out_raster,
                                 layer.out_extra)
    torch.cuda.synchronize()
    assert torch.equal(layer.out_extra.view(torch.int16), want_x.view(torch.int16))
    if want_r is not None:
        assert torch.equal(layer.out_raster.view(torch.int16), want_r.view(torch.int16))
    log(f"  bit-identical to the workspace call ({layer.ws.numel()} bytes of scratch)")


def test_noalloc_matches_workspace_call_twice():
    big = workloads.Workload(name="noalloc_decode", T=64, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=4,
                             n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=71,
                             video_queries=False, n_decode=5)
    small = workloads.Workload(name="noalloc_text", T=16, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=4,
                               n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=72,
                               video_queries=False, n_text=6, text_kv=True)
    _noalloc_matches(big)
    _noalloc_matches(small)

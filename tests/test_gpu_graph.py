"""The path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing and records no memset inside a call, so a
decode step (selection, extra-row bitmap, decode attention, merge) and a whole
prefill (partition of Q, K, V with the mean keys, selection, attention) can be
captured once and replayed with new inputs copied into the captured buffers.
Every replay must equal, bit for bit, the eager call on the same inputs (the
kernels are deterministic), also with eager calls on the same buffers between
replays.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_harness import geometry, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _lists(layer, n_cubes, first_extra_off):
    """(counts, the extra rows' list entries up to each count) on the host."""
    cnt = layer.sel_count.cpu().numpy().copy()
    idx = layer.sel_idx.cpu().numpy()
    hq, R = cnt.shape
    lists = [idx[first_extra_off + (h * R + r) * n_cubes:][:cnt[h, r]].copy() for h in range(hq) for r in range(R)]
    return cnt, lists


def _same(a, b, what):
    ca, la = a[0], a[1]
    cb, lb = b[0], b[1]
    assert np.array_equal(ca, cb), f"{what}: counts differ"
    assert all(np.array_equal(x, y) for x, y in zip(la, lb)), f"{what}: lists differ"
    assert torch.equal(a[2], b[2]), f"{what}: outputs differ"


def test_decode_step_graph_replays_equal_eager_steps():
    from adaptive_cube_sparse_amd import AdasAttention
    wl = workloads.get("decode")
    log(f"case {wl.name}: decode step in a graph, {wl.n_q_heads} heads, {wl.T}x{wl.H}x{wl.W} cache")
    data = workloads.generate(wl)
    dev = torch.device("cuda:0")
    geom = geometry(wl)
    layer = AdasAttention(geom, torch.bfloat16, wl.p, has_video=False, n_extra=1, device=dev)
    layer.build_kv(to_dev(data["k"], dev), to_dev(data["v"], dev))
    qall = to_dev(data["q_text"], dev)
    qs = [qall[i:i + 1].contiguous() for i in range(4)]

    def snap():
        torch.cuda.synchronize()
        return _lists(layer, geom.n_cubes, 0) + (layer.out_extra.clone(),)

    eager = []
    for q in qs:
        layer.decode_step(q)
        eager.append(snap())
    q_static = torch.empty_like(qs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q_static.copy_(qs[0])
        layer.decode_step(q_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.decode_step(q_static)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, q in enumerate(qs):
            q_static.copy_(q)
            graph.replay()
            _same(snap(), eager[i], f"replay {rep} query {i}")
            j = (i + 1) % len(qs)
            layer.decode_step(qs[j])  # eager work on the same buffers between replays
            _same(snap(), eager[j], f"eager between replays, query {j}")
    log("  12 replays and 12 eager steps between them: bit-identical to the eager steps")


def test_prefill_graph_replays_equal_eager_calls():
    from adaptive_cube_sparse_amd import AdasAttention
    # cubes of 32 tokens (register-staged key blocks) and causal text keys
    wl = workloads.get("tiny").replace(dtype="bf16", n_text=6, text_kv=True, name="tiny_graph")
    log(f"case {wl.name}: whole prefill in a graph (partition, mean keys, selection, attention)")
    dev = torch.device("cuda:0")
    n_extra = wl.n_text
    layer = AdasAttention(geometry(wl), torch.bfloat16, wl.p, has_video=True, n_extra=n_extra,
                          n_text_kv=n_extra, device=dev)
    inputs = []
    for seed in (11, 12, 13):
        d = workloads.generate(wl.replace(seed=seed))
        inputs.append({k: to_dev(d[k], dev) for k in ("q", "k", "v", "q_text", "k_text", "v_text")})

    def run(x):
        layer.forward(x["q"], x["k"], x["v"], x["q_text"], x["k_text"], x["v_text"])

    def snap():
        torch.cuda.synchronize()
        return (layer.sel_count.cpu().numpy().copy(), None,
                torch.cat([layer.out_raster.flatten(), layer.out_extra.flatten()]).clone())

    eager = []
    for x in inputs:
        run(x)
        eager.append(snap())
    static = {k: torch.empty_like(v) for k, v in inputs[0].items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in static:
            static[k].copy_(inputs[0][k])
        run(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(static)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, x in enumerate(inputs):
            for k in static:
                static[k].copy_(x[k])
            graph.replay()
            got = snap()
            assert np.array_equal(got[0], eager[i][0]), f"replay {rep} input {i}: counts differ"
            assert torch.equal(got[2], eager[i][2]), f"replay {rep} input {i}: outputs differ"
            j = (i + 1) % len(inputs)
            run(inputs[j])
            got = snap()
            assert torch.equal(got[2], eager[j][2]), f"eager between replays, input {j}: outputs differ"
    log("  9 replays and 9 eager calls between them: bit-identical to the eager calls")

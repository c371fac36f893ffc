"""CPU checks of the C ABI: the library loads, exports every symbol declared
in include/adas.h and include/adas_ffn.h, sizes buffers by the closed forms, and rejects invalid
arguments on the host before any launch (no GPU needed; no compute call)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "adaptive_cube_sparse_amd", "libadas.so")
HEADERS = [os.path.join(ROOT, "include", h) for h in ("adas.h", "adas_ffn.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libadas.so not built")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(adas_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) == set(L.EXPORTS)


def test_probes_reject_invalid_arguments_on_host():
    import ctypes
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    fl = ctypes.c_double(0.0)
    assert lib.adas_probe_mfma(0, 10, ctypes.c_void_p(16), ctypes.byref(fl), None) == L.ADAS_ERR_VALUE
    assert lib.adas_probe_mfma(8, 0, ctypes.c_void_p(16), ctypes.byref(fl), None) == L.ADAS_ERR_VALUE
    assert lib.adas_probe_mfma(8, 10, None, ctypes.byref(fl), None) == L.ADAS_ERR_NULL
    assert lib.adas_probe_hbm_read(None, 1024, ctypes.c_void_p(16), 0, None) == L.ADAS_ERR_NULL
    assert lib.adas_probe_hbm_read(ctypes.c_void_p(16), 1000, ctypes.c_void_p(16), 0, None) == L.ADAS_ERR_SHAPE
    assert lib.adas_probe_hbm_copy(ctypes.c_void_p(16), ctypes.c_void_p(16), 0, 0, None) == L.ADAS_ERR_SHAPE
    assert lib.adas_probe_hbm_copy(ctypes.c_void_p(16), None, 1024, 0, None) == L.ADAS_ERR_NULL
    assert lib.adas_probe_attn_mix(0, 10, 0, None, 0, ctypes.c_void_p(16), ctypes.byref(fl), None) == L.ADAS_ERR_VALUE
    assert lib.adas_probe_attn_mix(8, 10, 2, None, 0, ctypes.c_void_p(16), ctypes.byref(fl), None) == L.ADAS_ERR_VALUE
    assert lib.adas_probe_attn_mix(8, 10, 1, None, 4 << 20, ctypes.c_void_p(16), ctypes.byref(fl),
                                   None) == L.ADAS_ERR_NULL
    assert lib.adas_probe_attn_mix(8, 10, 1, ctypes.c_void_p(16), 1 << 20, ctypes.c_void_p(16), ctypes.byref(fl),
                                   None) == L.ADAS_ERR_SHAPE


def _geom(**kw):
    import adaptive_cube_sparse_amd._lib as L
    base = dict(T=8, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=6, n_kv_heads=2, head_dim=128)
    base.update(kw)
    g = L._Geom(**base)
    return g


def test_version_and_status_strings():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    assert lib.adas_version().decode() == "0.1"
    for s in range(8):
        assert lib.adas_status_string(s).decode().startswith("ADAS_")


def test_capacity_and_workspace_closed_forms():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _geom()
    N, S, Nc, Hq = 8 * 16 * 16, 64, 32, 6
    capv = S * Nc * (Nc - 1) // 2
    assert lib.adas_sel_capacity(ctypes.byref(g), 1, 0) == Hq * capv
    assert lib.adas_sel_capacity(ctypes.byref(g), 1, 5) == Hq * capv + Hq * 5 * Nc
    assert lib.adas_sel_capacity(ctypes.byref(g), 0, 5) == Hq * 5 * Nc
    # the selection keeps its logits on chip and needs no workspace ...
    assert lib.adas_workspace_bytes(ctypes.byref(g), L.ADAS_BF16, L.ADAS_WS_SELECT, 1, 0) == 0
    assert lib.adas_workspace_bytes(ctypes.byref(g), L.ADAS_F32, L.ADAS_WS_SELECT, 1, 0) == 0
    assert lib.adas_workspace_bytes(ctypes.byref(g), L.ADAS_BF16, L.ADAS_WS_SELECT, 0, 3) == 0
    # ... except extra rows over more than 1024 cubes (bf16): their float32 logits
    big = _geom(T=64, H=64, W=64)  # 16 x 16 x 16 = 4096 cubes
    assert lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_SELECT, 0, 3) == 6 * 3 * 4096 * 4
    assert lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_F32, L.ADAS_WS_SELECT, 0, 3) == 0
    assert lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_SELECT, 1, 0) == 0
    # prefill without extra rows needs no attention workspace
    assert lib.adas_workspace_bytes(ctypes.byref(g), L.ADAS_BF16, L.ADAS_WS_ATTN, 1, 0) == 0
    bad = _geom(ct=3)
    assert lib.adas_sel_capacity(ctypes.byref(bad), 1, 0) == -1


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _select(lib, g, **kw):
    import adaptive_cube_sparse_amd._lib as L
    args = dict(dtype=L.ADAS_BF16, q_cube=FAKE, n_extra=0, q_extra=None, kbar=FAKE, p=0.7,
                sel_count=FAKE, sel_idx=FAKE, cap=1 << 40, ws=FAKE, ws_bytes=1 << 40)
    args.update(kw)
    return lib.adas_select_topp(ctypes.byref(g) if g is not None else None, args["dtype"],
                                args["q_cube"], args["n_extra"], args["q_extra"], args["kbar"],
                                args["p"], args["sel_count"], args["sel_idx"], args["cap"],
                                args["ws"], args["ws_bytes"], None)


def test_select_rejects_invalid_arguments_on_host():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _geom()
    assert _select(lib, None) == L.ADAS_ERR_NULL
    for p in (0.0, -0.1, 1.0001, float("nan")):
        assert _select(lib, g, p=p) == L.ADAS_ERR_VALUE
    assert "p must be" in lib.adas_last_error().decode()
    assert _select(lib, _geom(ct=3)) == L.ADAS_ERR_SHAPE
    assert _select(lib, _geom(head_dim=96)) == L.ADAS_ERR_SHAPE
    assert _select(lib, _geom(n_q_heads=5)) == L.ADAS_ERR_SHAPE       # Hkv must divide Hq
    assert _select(lib, g, dtype=7) == L.ADAS_ERR_DTYPE
    assert _select(lib, g, q_cube=None) == L.ADAS_ERR_SHAPE           # no rows at all
    assert _select(lib, g, n_extra=3, q_extra=None) == L.ADAS_ERR_NULL
    assert _select(lib, g, kbar=None) == L.ADAS_ERR_NULL
    assert _select(lib, g, cap=10) == L.ADAS_ERR_CAPACITY
    big = _geom(T=64, H=64, W=64)  # 4096 cubes: extra rows need a logit workspace
    assert _select(lib, big, q_cube=None, n_extra=3, q_extra=FAKE, ws=None, ws_bytes=0) == L.ADAS_ERR_WORKSPACE
    assert _select(lib, big, q_cube=None, n_extra=3, q_extra=FAKE, ws_bytes=6 * 3 * 4096 * 4 - 1) == L.ADAS_ERR_WORKSPACE
    big = _geom(T=8, H=16, W=16 * 9, ct=1, ch=1, cw=4)               # 9216 cubes > 4096
    assert _select(lib, big) == L.ADAS_ERR_SHAPE
    # head_map entries must name an existing KV head
    hm = (ctypes.c_int32 * 6)(0, 1, 0, 1, 2, 0)
    g2 = _geom()
    g2.head_map = ctypes.cast(hm, ctypes.POINTER(ctypes.c_int32))
    assert _select(lib, g2) == L.ADAS_ERR_VALUE


def test_decode_step_workspace_and_host_validation():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    big = _geom(T=64, H=64, W=64)  # 4096 cubes: the split selection, the decode kernel
    n = 1
    attn = lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_ATTN, 0, n)
    sel = lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_SELECT, 0, n)
    dec = lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_DECODE, 0, n)
    assert attn > 0 and sel == 6 * n * 4096 * 4
    # the attention's part of a decode plan (no text keys: the decode kernel, about one workgroup per CU,
    # 256 / Hkv = 128 chunks of 32 cubes): the extra-row bitmap (128 words per row) and one partial row
    # (max, sum, d outputs) per (KV head, 32-row slot, chunk); then the selection's logits
    bitmap = 6 * n * 128 * 4
    partials = 2 * 32 * 128 * (128 + 2) * 4
    attn_decode = ((bitmap + 255) // 256) * 256 + partials
    assert dec == ((attn_decode + 255) // 256) * 256 + sel
    assert dec < attn + sel   # ADAS_WS_ATTN also covers the text-key plan (union tiles)
    assert lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_DECODE, 1, n) == 0  # no video rows
    assert lib.adas_workspace_bytes(ctypes.byref(big), L.ADAS_BF16, L.ADAS_WS_DECODE, 0, 0) == 0

    def step(g, **kw):
        a = dict(dtype=L.ADAS_BF16, n=n, q=FAKE, kbar=FAKE, k=FAKE, v=FAKE, p=0.7, cnt=FAKE, idx=FAKE,
                 cap=1 << 40, out=FAKE, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return lib.adas_decode_step(ctypes.byref(g) if g is not None else None, a["dtype"], a["n"], a["q"],
                                    a["kbar"], a["k"], a["v"], a["p"], a["cnt"], a["idx"], a["cap"], a["out"],
                                    a["ws"], a["ws_bytes"], None)
    assert step(None) == L.ADAS_ERR_NULL
    assert step(big, n=0) == L.ADAS_ERR_SHAPE
    for p in (0.0, 1.5, float("nan")):
        assert step(big, p=p) == L.ADAS_ERR_VALUE
    for k in ("q", "kbar", "k", "v", "cnt", "idx", "out"):
        assert step(big, **{k: None}) == L.ADAS_ERR_NULL
    assert step(big, dtype=9) == L.ADAS_ERR_DTYPE
    assert step(big, cap=6 * 4096 - 1) == L.ADAS_ERR_CAPACITY
    assert step(big, ws_bytes=dec - 1) == L.ADAS_ERR_WORKSPACE
    assert step(big, ws=None, ws_bytes=0) == L.ADAS_ERR_WORKSPACE
    assert step(_geom(ct=3)) == L.ADAS_ERR_SHAPE


def test_topk_rejects_invalid_arguments_on_host():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _geom()

    def topk(k, **kw):
        a = dict(q_cube=FAKE, cap=1 << 40)
        a.update(kw)
        return lib.adas_select_topk(ctypes.byref(g), L.ADAS_BF16, a["q_cube"], 0, None, FAKE, k,
                                    FAKE, FAKE, a["cap"], FAKE, 1 << 40, None)
    for k in (0, -3):
        assert topk(k) == L.ADAS_ERR_VALUE
    assert "k must be" in lib.adas_last_error().decode()
    assert topk(4, cap=10) == L.ADAS_ERR_CAPACITY
    assert topk(4, q_cube=None) == L.ADAS_ERR_SHAPE


def test_attention_and_partition_reject_invalid_arguments_on_host():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _geom()
    # partition: null buffers, bad head count, bad dtype
    T, VT = L.ADAS_LAYOUT_TOKENS, L.ADAS_LAYOUT_VT
    assert lib.adas_cube_partition(ctypes.byref(g), L.ADAS_BF16, 2, T, None, FAKE, None, None) == L.ADAS_ERR_NULL
    assert lib.adas_cube_partition(ctypes.byref(g), L.ADAS_BF16, 2, VT, FAKE, None, None, None) == L.ADAS_ERR_NULL
    assert lib.adas_cube_partition(ctypes.byref(g), L.ADAS_BF16, 0, T, FAKE, FAKE, None, None) == L.ADAS_ERR_SHAPE
    assert lib.adas_cube_partition(ctypes.byref(g), 9, 2, T, FAKE, FAKE, None, None) == L.ADAS_ERR_DTYPE
    assert lib.adas_cube_partition(ctypes.byref(g), L.ADAS_BF16, 2, 5, FAKE, FAKE, None, None) == L.ADAS_ERR_VALUE
    assert "layout" in lib.adas_last_error().decode()
    assert lib.adas_cube_mean_keys(ctypes.byref(g), L.ADAS_BF16, None, FAKE, None) == L.ADAS_ERR_NULL
    assert lib.adas_cube_partition_keys(ctypes.byref(g), L.ADAS_BF16, FAKE, FAKE, None, None,
                                        None) == L.ADAS_ERR_NULL
    assert lib.adas_cube_partition_keys(ctypes.byref(g), 9, FAKE, FAKE, None, FAKE, None) == L.ADAS_ERR_DTYPE

    def attn(**kw):
        a = dict(q_cube=FAKE, k=FAKE, v=FAKE, n_extra=0, n_text_kv=0, q_extra=None, kt=None, vt=None,
                 cnt=FAKE, idx=FAKE, out=FAKE, out_x=None, ws=None, ws_bytes=0)
        a.update(kw)
        return lib.adas_sparse_attn_fwd(ctypes.byref(g), L.ADAS_BF16, a["q_cube"], a["k"], a["v"],
                                        a["n_extra"], a["n_text_kv"], a["q_extra"], a["kt"], a["vt"],
                                        a["cnt"], a["idx"], a["out"], a["out_x"], a["ws"],
                                        a["ws_bytes"], None)
    assert attn(k=None) == L.ADAS_ERR_NULL
    assert attn(out=None) == L.ADAS_ERR_NULL
    assert attn(n_extra=4, q_extra=FAKE, out_x=None) == L.ADAS_ERR_NULL
    assert attn(n_extra=4, n_text_kv=3, q_extra=FAKE, out_x=FAKE) == L.ADAS_ERR_SHAPE
    assert attn(n_extra=4, n_text_kv=4, q_extra=FAKE, out_x=FAKE) == L.ADAS_ERR_NULL  # no text K/V
    assert attn(q_cube=None) == L.ADAS_ERR_SHAPE
    # decode rows split across cube chunks need a workspace
    need = lib.adas_workspace_bytes(ctypes.byref(g), L.ADAS_BF16, L.ADAS_WS_ATTN, 0, 2)
    assert need > 0
    assert attn(q_cube=None, out=None, n_extra=2, q_extra=FAKE, out_x=FAKE) == L.ADAS_ERR_WORKSPACE


def test_backward_rejects_invalid_arguments_on_host():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _geom()  # cubes of 64 tokens

    def bwd(geom=g, **kw):
        a = dict(q_cube=FAKE, n_extra=0, q_extra=None, out_x=None, dout_x=None, dq_x=None, ntk=0, kt=None,
                 vt=None, dkt=None, dvt=None, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return lib.adas_sparse_attn_bwd(ctypes.byref(geom), L.ADAS_BF16, a["q_cube"], FAKE, FAKE, FAKE,
                                        a["n_extra"], a["q_extra"], FAKE, FAKE, FAKE, a["out_x"], FAKE, FAKE,
                                        a["dout_x"], FAKE, a["dq_x"], FAKE, FAKE, a["ntk"], a["kt"], a["vt"],
                                        a["dkt"], a["dvt"], a["ws"], a["ws_bytes"], None)
    text = dict(n_extra=4, q_extra=FAKE, out_x=FAKE, dout_x=FAKE, dq_x=FAKE)
    assert bwd(**text, ntk=3) == L.ADAS_ERR_VALUE               # text keys must match the extra rows
    assert "n_text_kv" in lib.adas_last_error().decode()
    assert bwd(**text, ntk=4, kt=FAKE, vt=FAKE, dkt=None, dvt=FAKE) == L.ADAS_ERR_NULL
    assert bwd(**text, ntk=4, kt=None, vt=FAKE, dkt=FAKE, dvt=FAKE) == L.ADAS_ERR_NULL
    assert bwd(ntk=1) == L.ADAS_ERR_VALUE                        # no extra rows, no text keys
    assert bwd(ws=None) == L.ADAS_ERR_WORKSPACE
    assert bwd(geom=_geom(ct=2, ch=8, cw=8)) == L.ADAS_ERR_SHAPE  # cubes of 128: disabled
    assert bwd(q_cube=None) == L.ADAS_ERR_SHAPE                  # no rows at all


def _ffn_geom(**kw):
    import adaptive_cube_sparse_amd._lib as L
    base = dict(T=4, H=8, W=8, ct=2, ch=4, cw=4, hidden=256, inter=384)
    base.update(kw)
    return L._FfnGeom(**base)


def test_ffn_workspace_closed_form_and_host_validation():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _ffn_geom()
    rows = (256 + 5 + 255) // 256 * 256
    assert lib.adas_ffn_workspace_bytes(ctypes.byref(g), 5) == rows * 384 * 2 + rows * 256 * 4 + 256
    FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails on the host
    def sel(p=0.7, **kw):
        gg = _ffn_geom(**kw)
        return lib.adas_ffn_select(ctypes.byref(gg), FAKE, p, FAKE, FAKE, FAKE, FAKE, None)
    for bad in (0.0, -0.1, 1.5, float("nan")):
        assert sel(bad) == L.ADAS_ERR_VALUE
    assert sel(hidden=200) == L.ADAS_ERR_SHAPE
    assert sel(ct=3) == L.ADAS_ERR_SHAPE
    assert sel(T=8, H=8, W=8, ct=8, ch=8, cw=8) == L.ADAS_ERR_SHAPE  # S = 512 > ADAS_FFN_MAX_S
    assert lib.adas_ffn_select(ctypes.byref(g), None, 0.7, FAKE, FAKE, FAKE, FAKE, None) == L.ADAS_ERR_NULL
    def fwd(ws_bytes, inter=384, n_text=0, x_text=None):
        gg = _ffn_geom(inter=inter)
        return lib.adas_ffn_fwd(ctypes.byref(gg), FAKE, n_text, x_text, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, ws_bytes, None)
    need = lib.adas_ffn_workspace_bytes(ctypes.byref(g), 0)
    assert fwd(need - 1) == L.ADAS_ERR_WORKSPACE
    assert fwd(need, inter=320) == L.ADAS_ERR_SHAPE
    assert fwd(need, n_text=3) == L.ADAS_ERR_NULL


def test_cache_geometry_and_append_validation():
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails on the host
    g = _geom(T=8, cache_T=12)
    # cache_T must be 0 or a multiple of ct that is >= T
    for bad in (4, 10):
        gb = _geom(T=8, cache_T=bad)
        assert lib.adas_sel_capacity(ctypes.byref(gb), 0, 1) == -1
    assert lib.adas_sel_capacity(ctypes.byref(g), 0, 1) > 0
    # running sums: Hkv * nH * nW * d doubles
    assert lib.adas_cache_sum_bytes(ctypes.byref(g)) == 2 * 4 * 4 * 128 * 8
    def app(t0, n, dtype=None):
        return lib.adas_cache_append(ctypes.byref(g), L.ADAS_BF16 if dtype is None else dtype, t0, n,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert app(0, 0) == L.ADAS_ERR_SHAPE
    assert app(10, 3) == L.ADAS_ERR_SHAPE          # past the capacity of 12 frames
    assert app(-1, 2) == L.ADAS_ERR_SHAPE
    assert app(0, 4, L.ADAS_F32) == L.ADAS_ERR_DTYPE
    assert lib.adas_cache_append(ctypes.byref(g), L.ADAS_BF16, 0, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None) == L.ADAS_ERR_NULL


def test_noalloc_rejects_oversized_scratch_on_host():
    """A call whose attention scratch exceeds ADAS_NOALLOC_SCRATCH_BYTES is
    refused before anything is launched (pointers are never dereferenced on
    the host): 64 decode rows x 28 heads over 4096 cubes need about 68 MB of
    chunk partials."""
    import ctypes
    import adaptive_cube_sparse_amd._lib as L
    lib = L.load()
    g = _geom(T=1024, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=28, n_kv_heads=4, head_dim=128)
    need = lib.adas_workspace_bytes(ctypes.byref(g), L.ADAS_BF16, L.ADAS_WS_ATTN, 0, 64)
    assert need > L.ADAS_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(256)
    st = lib.adas_sparse_attn_fwd_noalloc(ctypes.byref(g), L.ADAS_BF16, None, p, p, 64, 0, p, None, None,
                                          p, p, None, p, None)
    assert st == L.ADAS_ERR_WORKSPACE
    assert b"allocation-free" in lib.adas_last_error()
    # invalid geometry is reported as by adas_sparse_attn_fwd
    g.head_dim = 96
    assert lib.adas_sparse_attn_fwd_noalloc(ctypes.byref(g), L.ADAS_BF16, None, p, p, 1, 0, p, None, None,
                                            p, p, None, p, None) == L.ADAS_ERR_SHAPE

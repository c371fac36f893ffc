"""ctypes binding of libadas (include/adas.h, include/adas_ffn.h).

Argument marshalling only: every function here checks tensor dtypes, devices
and shapes, turns tensors into raw pointers and calls the C entry point of
the same name on the current HIP stream.  No step of the computation runs in
Python.  If the compiled library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libadas.so")

ADAS_OK, ADAS_ERR_NULL, ADAS_ERR_SHAPE, ADAS_ERR_VALUE, ADAS_ERR_DTYPE, \
    ADAS_ERR_WORKSPACE, ADAS_ERR_CAPACITY, ADAS_ERR_HIP = range(8)
ADAS_BF16, ADAS_F32 = 0, 1
ADAS_WS_SELECT, ADAS_WS_ATTN, ADAS_WS_BWD, ADAS_WS_DECODE = 0, 1, 2, 3
ADAS_LAYOUT_TOKENS, ADAS_LAYOUT_VT = 0, 1
ADAS_MAX_HEADS = 128
ADAS_MAX_CUBES = 4096
ADAS_FFN_MAX_S = 256
ADAS_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "adas_cube_partition", "adas_cube_mean_keys", "adas_select_topp", "adas_select_topk",
    "adas_sparse_attn_fwd", "adas_workspace_bytes", "adas_sel_capacity",
    "adas_status_string", "adas_last_error", "adas_version",
    "adas_ffn_select", "adas_ffn_fwd", "adas_ffn_workspace_bytes",
    "adas_cache_append", "adas_cache_sum_bytes", "adas_sparse_attn_fwd_lse", "adas_sparse_attn_bwd",
    "adas_probe_mfma", "adas_probe_hbm_read", "adas_probe_hbm_copy", "adas_sparse_attn_fwd_noalloc",
    "adas_cube_partition_keys", "adas_probe_attn_mix", "adas_decode_step",
)


class AdasError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "W", "ct", "ch", "cw", "n_q_heads", "n_kv_heads", "head_dim")] + \
               [("head_map", ctypes.POINTER(ctypes.c_int32)), ("cache_T", ctypes.c_int32)]


class _FfnGeom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "W", "ct", "ch", "cw", "hidden", "inter")]


_lib = None


def load() -> ctypes.CDLL:
    """Load libadas.so (built in-tree); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libadas.so not found at {LIB_PATH}; build it with "
                          f"`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    gp = ctypes.POINTER(_Geom)
    fgp = ctypes.POINTER(_FfnGeom)
    f64 = ctypes.c_double
    sig = {
        "adas_cube_partition": (i32, [gp, i32, i32, i32, vp, vp, vp, vp]),
        "adas_cube_mean_keys": (i32, [gp, i32, vp, vp, vp]),
        "adas_cube_partition_keys": (i32, [gp, i32, vp, vp, vp, vp, vp]),
        "adas_select_topp": (i32, [gp, i32, vp, i32, vp, vp, f32, vp, vp, i64, vp, sz, vp]),
        "adas_select_topk": (i32, [gp, i32, vp, i32, vp, vp, i32, vp, vp, i64, vp, sz, vp]),
        "adas_sparse_attn_fwd": (i32, [gp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                       vp, vp, sz, vp]),
        "adas_workspace_bytes": (sz, [gp, i32, i32, i32, i32]),
        "adas_sel_capacity": (i64, [gp, i32, i32]),
        "adas_status_string": (ctypes.c_char_p, [i32]),
        "adas_last_error": (ctypes.c_char_p, []),
        "adas_version": (ctypes.c_char_p, []),
        "adas_ffn_select": (i32, [fgp, vp, f64, vp, vp, vp, vp, vp]),
        "adas_ffn_fwd": (i32, [fgp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "adas_ffn_workspace_bytes": (sz, [fgp, i32]),
        "adas_cache_append": (i32, [gp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]),
        "adas_cache_sum_bytes": (sz, [gp]),
        "adas_sparse_attn_fwd_lse": (i32, [gp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, sz, vp]),
        "adas_sparse_attn_bwd": (i32, [gp, i32, vp, vp, vp, vp, i32] + [vp] * 12 + [i32, vp, vp, vp, vp]
                                 + [vp, sz, vp]),
        "adas_sparse_attn_fwd_noalloc": (i32, [gp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                               vp, vp]),
        "adas_probe_mfma": (i32, [i32, i32, vp, ctypes.POINTER(f64), vp]),
        "adas_probe_hbm_read": (i32, [vp, i64, vp, i32, vp]),
        "adas_probe_hbm_copy": (i32, [vp, vp, i64, i32, vp]),
        "adas_probe_attn_mix": (i32, [i32, i32, i32, vp, i64, vp, ctypes.POINTER(f64), vp]),
        "adas_decode_step": (i32, [gp, i32, i32, vp, vp, vp, vp, f32, vp, vp, i64, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# geometry
# ---------------------------------------------------------------------------
@dataclass
class Geometry:
    """Frame grid T x H x W, cube extents (ct, ch, cw) = (t, h, w), heads."""
    T: int
    H: int
    W: int
    ct: int
    ch: int
    cw: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    head_map: Optional[Sequence[int]] = None
    cache_T: int = 0   # frames per head allocated in cube-layout buffers (0: T)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def NS(self) -> int:
        """Tokens per head of a cube-layout buffer."""
        return (self.cache_T or self.T) * self.H * self.W

    @property
    def S(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def n_cubes(self) -> int:
        return self.N // self.S

    def _c(self):
        g = _Geom(self.T, self.H, self.W, self.ct, self.ch, self.cw, self.n_q_heads,
                  self.n_kv_heads, self.head_dim)
        g.cache_T = self.cache_T
        keep = None
        if self.head_map is not None:
            keep = (ctypes.c_int32 * len(self.head_map))(*[int(x) for x in self.head_map])
            g.head_map = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
        return g, keep


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ADAS_BF16
    if t.dtype == torch.float32:
        return ADAS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shape(t: Optional[torch.Tensor], shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != ADAS_OK:
        lib = load()
        msg = lib.adas_last_error().decode() or lib.adas_status_string(status).decode()
        raise AdasError(status, where, msg)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def adas_cube_partition(geom: Geometry, x_raster: torch.Tensor, x_cube: torch.Tensor,
                        perm: Optional[torch.Tensor] = None, stream=None,
                        layout: int = ADAS_LAYOUT_TOKENS) -> None:
    """x_raster [N][nh][d] -> x_cube [nh][N][d] (ADAS_LAYOUT_TOKENS) or
    [nh][Nc][d][S] (ADAS_LAYOUT_VT, the value layout of the attention), plus
    perm [N] int32."""
    lib = load()
    N, nh, d = x_raster.shape
    if layout == ADAS_LAYOUT_VT:
        _shape(x_cube, (nh, geom.NS // geom.S, d, geom.S), "x_cube")
    else:
        _shape(x_cube, (nh, geom.NS, d), "x_cube")
    _shape(perm, (N,), "perm")
    g, keep = geom._c()
    st = lib.adas_cube_partition(ctypes.byref(g), _dtype_code(x_raster), nh, int(layout),
                                 _ptr(x_raster, name="x_raster"),
                                 _ptr(x_cube, x_raster.dtype, "x_cube"),
                                 _ptr(perm, torch.int32, "perm"), _stream(stream))
    _check(st, "adas_cube_partition")


def adas_cube_mean_keys(geom: Geometry, k_cube: torch.Tensor, kbar: torch.Tensor,
                        stream=None) -> None:
    """k_cube [Hkv][N][d] -> kbar [Hkv][Nc][d] float32."""
    lib = load()
    _shape(k_cube, (geom.n_kv_heads, geom.NS, geom.head_dim), "k_cube")
    _shape(kbar, (geom.n_kv_heads, geom.NS // geom.S, geom.head_dim), "kbar")
    g, keep = geom._c()
    st = lib.adas_cube_mean_keys(ctypes.byref(g), _dtype_code(k_cube), _ptr(k_cube, name="k_cube"),
                                 _ptr(kbar, torch.float32, "kbar"), _stream(stream))
    _check(st, "adas_cube_mean_keys")


def adas_cube_partition_keys(geom: Geometry, k_raster: torch.Tensor, k_cube: torch.Tensor,
                             perm: Optional[torch.Tensor], kbar: torch.Tensor, stream=None) -> None:
    """k_raster [N][Hkv][d] -> k_cube [Hkv][N][d], perm [N] int32 and kbar
    [Hkv][Nc][d] float32 in one pass over K."""
    lib = load()
    _shape(k_raster, (geom.N, geom.n_kv_heads, geom.head_dim), "k_raster")
    _shape(k_cube, (geom.n_kv_heads, geom.NS, geom.head_dim), "k_cube")
    _shape(perm, (geom.N,), "perm")
    _shape(kbar, (geom.n_kv_heads, geom.NS // geom.S, geom.head_dim), "kbar")
    g, keep = geom._c()
    st = lib.adas_cube_partition_keys(ctypes.byref(g), _dtype_code(k_raster), _ptr(k_raster, name="k_raster"),
                                      _ptr(k_cube, k_raster.dtype, "k_cube"), _ptr(perm, torch.int32, "perm"),
                                      _ptr(kbar, torch.float32, "kbar"), _stream(stream))
    _check(st, "adas_cube_partition_keys")


def _select(fn, name, geom, q_cube, q_extra, kbar, arg, sel_count, sel_idx, ws, stream):
    lib = load()
    ref = q_cube if q_cube is not None else q_extra
    n_extra = 0 if q_extra is None else q_extra.shape[0]
    _shape(q_cube, (geom.n_q_heads, geom.NS, geom.head_dim), "q_cube")
    if q_extra is not None:
        _shape(q_extra, (n_extra, geom.n_q_heads, geom.head_dim), "q_extra")
    rows = (geom.N if q_cube is not None else 0) + n_extra
    _shape(sel_count, (geom.n_q_heads, rows), "sel_count")
    g, keep = geom._c()
    st = getattr(lib, fn)(ctypes.byref(g), _dtype_code(ref), _ptr(q_cube, ref.dtype, "q_cube"),
                          n_extra, _ptr(q_extra, ref.dtype, "q_extra"),
                          _ptr(kbar, torch.float32, "kbar"), arg,
                          _ptr(sel_count, torch.int32, "sel_count"),
                          _ptr(sel_idx, torch.int32, "sel_idx"), sel_idx.numel(),
                          _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(),
                          _stream(stream))
    _check(st, name)


def adas_select_topp(geom: Geometry, q_cube: Optional[torch.Tensor], q_extra: Optional[torch.Tensor],
                     kbar: torch.Tensor, p: float, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                     ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Top-p cube sets for video rows (q_cube [Hq][N][d]) and extra rows
    (q_extra [n_extra][Hq][d]); see adas.h for the output layout."""
    _select("adas_select_topp", "adas_select_topp", geom, q_cube, q_extra, kbar, float(p),
            sel_count, sel_idx, ws, stream)


def adas_select_topk(geom: Geometry, q_cube: Optional[torch.Tensor], q_extra: Optional[torch.Tensor],
                     kbar: torch.Tensor, k: int, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                     ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Top-K cube sets (k most probable candidates); same layout as Top-p."""
    _select("adas_select_topk", "adas_select_topk", geom, q_cube, q_extra, kbar, int(k),
            sel_count, sel_idx, ws, stream)


def adas_sparse_attn_fwd(geom: Geometry, q_cube, k_cube, v_cube, q_extra, k_text, v_text,
                         sel_count, sel_idx, out_raster, out_extra,
                         ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Attention over selected cubes plus own cube (video rows) or selected
    cubes plus causal text (extra rows); see adas.h."""
    args = _attn_args(geom, q_cube, k_cube, v_cube, q_extra, k_text, v_text, sel_count, sel_idx,
                      out_raster, out_extra)
    st = load().adas_sparse_attn_fwd(*args, _ptr(ws, name="ws"),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "adas_sparse_attn_fwd")


def adas_sparse_attn_fwd_noalloc(geom: Geometry, q_cube, k_cube, v_cube, q_extra, k_text, v_text,
                                 sel_count, sel_idx, out_raster, out_extra, stream=None) -> None:
    """adas_sparse_attn_fwd without a workspace: the library's per-GPU scratch
    array (ADAS_NOALLOC_SCRATCH_BYTES) takes its place; see adas.h."""
    args = _attn_args(geom, q_cube, k_cube, v_cube, q_extra, k_text, v_text, sel_count, sel_idx,
                      out_raster, out_extra)
    st = load().adas_sparse_attn_fwd_noalloc(*args, _stream(stream))
    _check(st, "adas_sparse_attn_fwd_noalloc")


def adas_decode_step(geom: Geometry, q_extra: torch.Tensor, kbar: torch.Tensor, k_cube: torch.Tensor,
                     v_cube: torch.Tensor, p: float, sel_count: torch.Tensor, sel_idx: torch.Tensor,
                     out_extra: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Selection and attention of n_extra query tokens over a built cache in
    one call (q_extra, out_extra [n_extra][Hq][d]); see adas.h."""
    n_extra = q_extra.shape[0]
    Hq, Hkv, d = geom.n_q_heads, geom.n_kv_heads, geom.head_dim
    _shape(q_extra, (n_extra, Hq, d), "q_extra")
    _shape(out_extra, (n_extra, Hq, d), "out_extra")
    _shape(k_cube, (Hkv, geom.NS, d), "k_cube")
    _shape(v_cube, (Hkv, geom.NS // geom.S, d, geom.S), "v_cube")  # ADAS_LAYOUT_VT
    _shape(sel_count, (Hq, n_extra), "sel_count")
    dt = q_extra.dtype
    g, keep = geom._c()
    st = load().adas_decode_step(ctypes.byref(g), _dtype_code(q_extra), n_extra, _ptr(q_extra, dt, "q_extra"),
                                 _ptr(kbar, torch.float32, "kbar"), _ptr(k_cube, dt, "k_cube"),
                                 _ptr(v_cube, dt, "v_cube"), float(p), _ptr(sel_count, torch.int32, "sel_count"),
                                 _ptr(sel_idx, torch.int32, "sel_idx"), sel_idx.numel(),
                                 _ptr(out_extra, dt, "out_extra"), _ptr(ws, name="ws"),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "adas_decode_step")


def _attn_args(geom: Geometry, q_cube, k_cube, v_cube, q_extra, k_text, v_text, sel_count, sel_idx,
               out_raster, out_extra):
    """Shape checks and the pointer arguments shared by the attention calls
    (geometry through out_extra)."""
    ref = q_cube if q_cube is not None else q_extra
    n_extra = 0 if q_extra is None else q_extra.shape[0]
    n_text_kv = 0 if k_text is None else k_text.shape[0]
    Hq, Hkv, d = geom.n_q_heads, geom.n_kv_heads, geom.head_dim
    _shape(q_cube, (Hq, geom.NS, d), "q_cube")
    _shape(k_cube, (Hkv, geom.NS, d), "k_cube")
    _shape(v_cube, (Hkv, geom.NS // geom.S, d, geom.S), "v_cube")  # ADAS_LAYOUT_VT
    _shape(out_raster, (geom.N, Hq, d), "out_raster")
    if n_extra:
        _shape(q_extra, (n_extra, Hq, d), "q_extra")
        _shape(out_extra, (n_extra, Hq, d), "out_extra")
    if n_text_kv:
        _shape(k_text, (n_text_kv, Hkv, d), "k_text")
        _shape(v_text, (n_text_kv, Hkv, d), "v_text")
    dt = ref.dtype
    g, keep = geom._c()   # byref(g) keeps g (and through it the head map) alive
    return (ctypes.byref(g), _dtype_code(ref), _ptr(q_cube, dt, "q_cube"), _ptr(k_cube, dt, "k_cube"),
            _ptr(v_cube, dt, "v_cube"), n_extra, n_text_kv, _ptr(q_extra, dt, "q_extra"),
            _ptr(k_text, dt, "k_text"), _ptr(v_text, dt, "v_text"),
            _ptr(sel_count, torch.int32, "sel_count"), _ptr(sel_idx, torch.int32, "sel_idx"),
            _ptr(out_raster, dt, "out_raster"), _ptr(out_extra, dt, "out_extra"))


def adas_cache_append(geom: Geometry, t0: int, k_new: torch.Tensor, v_new: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, kbar: torch.Tensor,
                      ksum: torch.Tensor, stream=None) -> None:
    """Append frames t0 .. t0 + n - 1 (k_new, v_new [n*H*W][Hkv][d], bf16) to a
    cube-layout KV cache sized for `geom` (T or cache_T frames); mean keys of
    completed cubes go to kbar.  ksum: adas_cache_sum_bytes() bytes kept
    between calls."""
    lib = load()
    hw = geom.H * geom.W
    if k_new.shape[0] % hw:
        raise ValueError("k_new must hold whole frames")
    n = k_new.shape[0] // hw
    Hkv, d = geom.n_kv_heads, geom.head_dim
    cap = geom.cache_T or geom.T
    ns = cap * hw
    _shape(k_new, (n * hw, Hkv, d), "k_new")
    _shape(v_new, (n * hw, Hkv, d), "v_new")
    _shape(k_cache, (Hkv, ns, d), "k_cache")
    _shape(v_cache, (Hkv, ns // geom.S, d, geom.S), "v_cache")
    _shape(kbar, (Hkv, ns // geom.S, d), "kbar")
    g, keep = geom._c()
    need = lib.adas_cache_sum_bytes(ctypes.byref(g))
    if ksum.numel() * ksum.element_size() < need:
        raise ValueError(f"ksum holds {ksum.numel() * ksum.element_size()} bytes, needs {need}")
    bf = torch.bfloat16
    st = lib.adas_cache_append(ctypes.byref(g), ADAS_BF16, int(t0), n, _ptr(k_new, bf, "k_new"),
                               _ptr(v_new, bf, "v_new"), _ptr(k_cache, bf, "k_cache"),
                               _ptr(v_cache, bf, "v_cache"), _ptr(kbar, torch.float32, "kbar"),
                               _ptr(ksum, name="ksum"), _stream(stream))
    _check(st, "adas_cache_append")


def adas_cache_sum_bytes(geom: Geometry) -> int:
    lib = load()
    g, keep = geom._c()
    return int(lib.adas_cache_sum_bytes(ctypes.byref(g)))


def adas_sparse_attn_fwd_lse(geom: Geometry, q_cube, k_cube, v_cube, q_extra, k_text, v_text,
                             sel_count, sel_idx, out_raster, out_extra, lse,
                             ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """adas_sparse_attn_fwd that also writes each row's log-sum-exp to
    lse [Hq][rows] (float32)."""
    lib = load()
    ref = q_cube if q_cube is not None else q_extra
    n_extra = 0 if q_extra is None else q_extra.shape[0]
    n_text_kv = 0 if k_text is None else k_text.shape[0]
    Hq, Hkv, d = geom.n_q_heads, geom.n_kv_heads, geom.head_dim
    _shape(q_cube, (Hq, geom.NS, d), "q_cube")
    _shape(k_cube, (Hkv, geom.NS, d), "k_cube")
    _shape(v_cube, (Hkv, geom.NS // geom.S, d, geom.S), "v_cube")
    _shape(lse, tuple(sel_count.shape), "lse")
    dt = ref.dtype
    g, keep = geom._c()
    st = lib.adas_sparse_attn_fwd_lse(
        ctypes.byref(g), _dtype_code(ref), _ptr(q_cube, dt, "q_cube"), _ptr(k_cube, dt, "k_cube"),
        _ptr(v_cube, dt, "v_cube"), n_extra, n_text_kv, _ptr(q_extra, dt, "q_extra"),
        _ptr(k_text, dt, "k_text"), _ptr(v_text, dt, "v_text"),
        _ptr(sel_count, torch.int32, "sel_count"), _ptr(sel_idx, torch.int32, "sel_idx"),
        _ptr(out_raster, dt, "out_raster"), _ptr(out_extra, dt, "out_extra"), _ptr(lse, torch.float32, "lse"),
        _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "adas_sparse_attn_fwd_lse")


def adas_sparse_attn_bwd(geom: Geometry, q_cube, k_cube, v_tok, k_vt, q_extra, sel_count, sel_idx,
                         out_raster, out_extra, lse, dout_raster, dout_extra, dq_raster, dq_extra,
                         dk_raster, dv_raster, ws: torch.Tensor, stream=None, k_text=None, v_text=None,
                         dk_text=None, dv_text=None) -> None:
    """Gradients of the sparse attention with the selection held fixed; see
    adas.h (bf16 inputs, float32 gradients in raster order).  k_text / v_text
    [n_extra][Hkv][d]: the causal text keys of a text prefill, whose gradients
    go to dk_text / dv_text."""
    lib = load()
    n_extra = 0 if q_extra is None else q_extra.shape[0]
    Hq, Hkv, d = geom.n_q_heads, geom.n_kv_heads, geom.head_dim
    bf, f32 = torch.bfloat16, torch.float32
    _shape(q_cube, (Hq, geom.NS, d), "q_cube")
    _shape(k_cube, (Hkv, geom.NS, d), "k_cube")
    _shape(v_tok, (Hkv, geom.NS, d), "v_tok")
    _shape(k_vt, (Hkv, geom.NS // geom.S, d, geom.S), "k_vt")
    _shape(dk_raster, (geom.N, Hkv, d), "dk_raster")
    _shape(dv_raster, (geom.N, Hkv, d), "dv_raster")
    if q_cube is not None:
        _shape(dq_raster, (geom.N, Hq, d), "dq_raster")
        _shape(dout_raster, (geom.N, Hq, d), "dout_raster")
    if n_extra:
        _shape(dq_extra, (n_extra, Hq, d), "dq_extra")
        _shape(dout_extra, (n_extra, Hq, d), "dout_extra")
    n_text_kv = 0 if k_text is None else k_text.shape[0]
    if n_text_kv:
        for t, name in ((k_text, "k_text"), (v_text, "v_text"), (dk_text, "dk_text"), (dv_text, "dv_text")):
            _shape(t, (n_text_kv, Hkv, d), name)
    g, keep = geom._c()
    st = lib.adas_sparse_attn_bwd(
        ctypes.byref(g), ADAS_BF16, _ptr(q_cube, bf, "q_cube"), _ptr(k_cube, bf, "k_cube"), _ptr(v_tok, bf, "v_tok"),
        _ptr(k_vt, bf, "k_vt"), n_extra, _ptr(q_extra, bf, "q_extra"), _ptr(sel_count, torch.int32, "sel_count"),
        _ptr(sel_idx, torch.int32, "sel_idx"), _ptr(out_raster, bf, "out_raster"), _ptr(out_extra, bf, "out_extra"),
        _ptr(lse, f32, "lse"), _ptr(dout_raster, bf, "dout_raster"), _ptr(dout_extra, bf, "dout_extra"),
        _ptr(dq_raster, f32, "dq_raster"), _ptr(dq_extra, f32, "dq_extra"), _ptr(dk_raster, f32, "dk_raster"),
        _ptr(dv_raster, f32, "dv_raster"), n_text_kv, _ptr(k_text, bf, "k_text"), _ptr(v_text, bf, "v_text"),
        _ptr(dk_text, f32, "dk_text"), _ptr(dv_text, f32, "dv_text"), _ptr(ws, name="ws"),
        ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "adas_sparse_attn_bwd")


def adas_workspace_bytes(geom: Geometry, dtype: torch.dtype, kind: int, has_video: bool,
                         n_extra: int) -> int:
    lib = load()
    g, keep = geom._c()
    code = ADAS_BF16 if dtype == torch.bfloat16 else ADAS_F32
    return int(lib.adas_workspace_bytes(ctypes.byref(g), code, kind, int(has_video), n_extra))


def adas_sel_capacity(geom: Geometry, has_video: bool, n_extra: int) -> int:
    lib = load()
    g, keep = geom._c()
    return int(lib.adas_sel_capacity(ctypes.byref(g), int(has_video), n_extra))


def adas_version() -> str:
    return load().adas_version().decode()


# ---------------------------------------------------------------------------
# measurement helpers (peak probes; not part of the method)
# ---------------------------------------------------------------------------
def adas_probe_mfma(workgroups: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the MFMA-only loop; returns the dense bf16 FLOPs it issues."""
    lib = load()
    _shape(sink, (workgroups,), "sink")
    fl = ctypes.c_double(0.0)
    st = lib.adas_probe_mfma(int(workgroups), int(iters), _ptr(sink, torch.float32, "sink"), ctypes.byref(fl),
                             _stream(stream))
    _check(st, "adas_probe_mfma")
    return fl.value


def adas_probe_attn_mix(workgroups: int, iters: int, mix: bool, src: Optional[torch.Tensor], sink: torch.Tensor,
                        stream=None) -> float:
    """Launch the MFMA loop alone (mix False) or with the union attention's
    side work (mix True; src: a device buffer of at least 2 MiB); returns the
    dense bf16 FLOPs it issues."""
    lib = load()
    _shape(sink, (workgroups,), "sink")
    nbytes = 0 if src is None else src.numel() * src.element_size()
    fl = ctypes.c_double(0.0)
    st = lib.adas_probe_attn_mix(int(workgroups), int(iters), 1 if mix else 0,
                                 None if src is None else _ptr(src, name="src"), nbytes,
                                 _ptr(sink, torch.float32, "sink"), ctypes.byref(fl), _stream(stream))
    _check(st, "adas_probe_attn_mix")
    return fl.value


def adas_probe_hbm_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, stream=None) -> int:
    """Stream src once; returns the bytes read."""
    lib = load()
    nbytes = src.numel() * src.element_size()
    st = lib.adas_probe_hbm_read(_ptr(src, name="src"), nbytes, _ptr(sink, torch.int32, "sink"), int(workgroups),
                                 _stream(stream))
    _check(st, "adas_probe_hbm_read")
    return nbytes


def adas_probe_hbm_copy(src: torch.Tensor, dst: torch.Tensor, workgroups: int = 0, stream=None) -> int:
    """Copy src to dst; returns the bytes copied (each way)."""
    lib = load()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    st = lib.adas_probe_hbm_copy(_ptr(src, name="src"), _ptr(dst, name="dst"), nbytes, int(workgroups),
                                 _stream(stream))
    _check(st, "adas_probe_hbm_copy")
    return nbytes


# ---------------------------------------------------------------------------
# AdaS-FFN (include/adas_ffn.h)
# ---------------------------------------------------------------------------
@dataclass
class FfnGeometry:
    """Video grid T x H x W, cube extents (ct, ch, cw), model and FFN widths."""
    T: int
    H: int
    W: int
    ct: int
    ch: int
    cw: int
    hidden: int
    inter: int

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def S(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def n_cubes(self) -> int:
        return self.N // self.S

    @property
    def mask_words(self) -> int:
        return (self.S + 31) // 32

    def _c(self):
        return _FfnGeom(self.T, self.H, self.W, self.ct, self.ch, self.cw, self.hidden, self.inter)


def adas_ffn_select(geom: FfnGeometry, x: torch.Tensor, p: float, act_count: torch.Tensor,
                    act_off: torch.Tensor, act_rows: torch.Tensor, act_mask: torch.Tensor,
                    stream=None) -> None:
    """Per-cube Top-p over token L2-norm shares: x [N][hidden] bf16 ->
    act_count [Nc], act_off [Nc+1], act_rows [N] int32, act_mask [Nc][words]."""
    lib = load()
    _shape(x, (geom.N, geom.hidden), "x")
    _shape(act_count, (geom.n_cubes,), "act_count")
    _shape(act_off, (geom.n_cubes + 1,), "act_off")
    _shape(act_rows, (geom.N,), "act_rows")
    _shape(act_mask, (geom.n_cubes, geom.mask_words), "act_mask")
    g = geom._c()
    st = lib.adas_ffn_select(ctypes.byref(g), _ptr(x, torch.bfloat16, "x"), float(p),
                             _ptr(act_count, torch.int32, "act_count"), _ptr(act_off, torch.int32, "act_off"),
                             _ptr(act_rows, torch.int32, "act_rows"), _ptr(act_mask, torch.int32, "act_mask"),
                             _stream(stream))
    _check(st, "adas_ffn_select")


def adas_ffn_fwd(geom: FfnGeometry, x: torch.Tensor, x_text: Optional[torch.Tensor], w_gate: torch.Tensor,
                 w_up: torch.Tensor, w_down: torch.Tensor, act_off: torch.Tensor, act_rows: torch.Tensor,
                 act_mask: torch.Tensor, y: torch.Tensor, y_text: Optional[torch.Tensor],
                 ws: torch.Tensor, stream=None) -> None:
    """FFN of the active tokens, mean compensation of the skipped ones, dense
    text tokens; see adas_ffn.h."""
    lib = load()
    n_text = 0 if x_text is None else x_text.shape[0]
    bf = torch.bfloat16
    _shape(x, (geom.N, geom.hidden), "x")
    _shape(y, (geom.N, geom.hidden), "y")
    _shape(w_gate, (geom.inter, geom.hidden), "w_gate")
    _shape(w_up, (geom.inter, geom.hidden), "w_up")
    _shape(w_down, (geom.hidden, geom.inter), "w_down")
    if n_text:
        _shape(x_text, (n_text, geom.hidden), "x_text")
        _shape(y_text, (n_text, geom.hidden), "y_text")
    g = geom._c()
    st = lib.adas_ffn_fwd(ctypes.byref(g), _ptr(x, bf, "x"), n_text, _ptr(x_text, bf, "x_text"),
                          _ptr(w_gate, bf, "w_gate"), _ptr(w_up, bf, "w_up"), _ptr(w_down, bf, "w_down"),
                          _ptr(act_off, torch.int32, "act_off"), _ptr(act_rows, torch.int32, "act_rows"),
                          _ptr(act_mask, torch.int32, "act_mask"), _ptr(y, bf, "y"), _ptr(y_text, bf, "y_text"),
                          _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "adas_ffn_fwd")


def adas_ffn_workspace_bytes(geom: FfnGeometry, n_text: int) -> int:
    lib = load()
    g = geom._c()
    return int(lib.adas_ffn_workspace_bytes(ctypes.byref(g), int(n_text)))

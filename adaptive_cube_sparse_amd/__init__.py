"""AdaS-Attn (AdaSpark adaptive cube-selective attention) and AdaS-FFN
(adaptive token-selective FFN) on MI355X.

The computation lives in libadas.so (hand-written HIP for gfx950, C ABI in
include/adas.h and include/adas_ffn.h).  This package is its Python binding
(``_lib``) plus ``AdasAttention``, which owns the device buffers of one layer
and chains the four library calls:

    cube partition (Q, K, V) -> cube mean keys -> Top-p (or Top-K) selection -> attention

``AdasFFN``, which chains the two AdaS-FFN calls:

    token selection per cube -> FFN of active tokens + mean compensation

and ``StreamingCache``, a video KV cache that grows frame by frame while
decode steps read its completed cubes.

Torch is used for device memory and streams only.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import (  # noqa: F401
    ADAS_BF16, ADAS_F32, ADAS_LAYOUT_TOKENS, ADAS_LAYOUT_VT, ADAS_WS_ATTN, ADAS_WS_SELECT,
    AdasError, FfnGeometry, Geometry, LIB_PATH,
    adas_ffn_fwd, adas_ffn_select, adas_ffn_workspace_bytes, adas_cache_append, adas_cache_sum_bytes,
    adas_sparse_attn_fwd_lse, adas_sparse_attn_bwd, ADAS_WS_BWD,
    adas_cube_mean_keys, adas_cube_partition, adas_cube_partition_keys, adas_select_topk, adas_select_topp,
    adas_sel_capacity,
    adas_sparse_attn_fwd, adas_version, adas_workspace_bytes, load, adas_sparse_attn_fwd_noalloc,
    adas_decode_step, ADAS_WS_DECODE,
)

__all__ = [
    "Geometry", "AdasAttention", "AdasError", "adas_cube_partition", "adas_cube_mean_keys",
    "adas_cube_partition_keys",
    "adas_select_topp", "adas_select_topk", "adas_sparse_attn_fwd", "adas_decode_step", "adas_workspace_bytes",
    "adas_sel_capacity",
    "adas_version", "load", "LIB_PATH",
    "FfnGeometry", "AdasFFN", "adas_ffn_select", "adas_ffn_fwd", "adas_ffn_workspace_bytes",
    "adas_cache_append", "adas_cache_sum_bytes", "StreamingCache",
    "adas_sparse_attn_fwd_lse", "adas_sparse_attn_bwd", "AdasAttentionGrad", "adas_sparse_attn_fwd_noalloc",
]


class AdasAttention:
    """Buffers and call sequence for one AdaS-Attn layer on one device.

    has_video: video query rows are present (prefill); False for decode.
    n_extra:   text / decode query tokens; n_text_kv: text K/V tokens
               (0 or n_extra).
    topk:      select the topk most probable cubes per row instead of Top-p.
    """

    def __init__(self, geom: Geometry, dtype: torch.dtype, p: float, has_video: bool = True,
                 n_extra: int = 0, n_text_kv: int = 0, device="cuda", topk: Optional[int] = None):
        load()
        self.geom, self.dtype, self.p = geom, dtype, float(p)
        self.topk = topk
        self.has_video, self.n_extra, self.n_text_kv = has_video, n_extra, n_text_kv
        g = geom
        dev = torch.device(device)
        e = dict(device=dev, dtype=dtype)
        self.k_cube = torch.empty((g.n_kv_heads, g.N, g.head_dim), **e)
        # values are kept cube-transposed (ADAS_LAYOUT_VT), the layout the attention reads
        self.v_cube = torch.empty((g.n_kv_heads, g.n_cubes, g.head_dim, g.S), **e)
        self.perm = torch.empty((g.N,), device=dev, dtype=torch.int32)
        self.kbar = torch.empty((g.n_kv_heads, g.n_cubes, g.head_dim), device=dev, dtype=torch.float32)
        self.q_cube = torch.empty((g.n_q_heads, g.N, g.head_dim), **e) if has_video else None
        self.out_raster = torch.empty((g.N, g.n_q_heads, g.head_dim), **e) if has_video else None
        self.out_extra = torch.empty((n_extra, g.n_q_heads, g.head_dim), **e) if n_extra else None
        rows = (g.N if has_video else 0) + n_extra
        self.sel_count = torch.empty((g.n_q_heads, rows), device=dev, dtype=torch.int32)
        cap = adas_sel_capacity(g, has_video, n_extra)
        if cap < 0:
            raise AdasError(2, "AdasAttention", "invalid geometry")
        self.sel_idx = torch.empty((max(cap, 1),), device=dev, dtype=torch.int32)
        wsb = adas_workspace_bytes(g, dtype, ADAS_WS_ATTN, has_video, n_extra)
        self.ws = torch.empty((max(wsb, 1),), device=dev, dtype=torch.uint8) if wsb else None
        wss = adas_workspace_bytes(g, dtype, ADAS_WS_SELECT, has_video, n_extra)
        self.ws_select = torch.empty((wss,), device=dev, dtype=torch.uint8) if wss else None

    # -- steps ---------------------------------------------------------------
    def build_kv(self, k_raster: torch.Tensor, v_raster: torch.Tensor, stream=None):
        """Partition K (token rows, with the cube mean keys in the same pass)
        and V (cube-transposed) into cube layout."""
        g = self.geom
        adas_cube_partition_keys(g, k_raster, self.k_cube, self.perm, self.kbar, stream)
        adas_cube_partition(g, v_raster, self.v_cube, None, stream, layout=ADAS_LAYOUT_VT)

    def partition_queries(self, q_raster: torch.Tensor, stream=None):
        adas_cube_partition(self.geom, q_raster, self.q_cube, None, stream)

    def select(self, q_extra: Optional[torch.Tensor] = None, p: Optional[float] = None, stream=None):
        if self.topk is not None and p is None:
            adas_select_topk(self.geom, self.q_cube, q_extra, self.kbar, self.topk,
                             self.sel_count, self.sel_idx, self.ws_select, stream)
            return
        adas_select_topp(self.geom, self.q_cube, q_extra, self.kbar, self.p if p is None else p,
                         self.sel_count, self.sel_idx, self.ws_select, stream)

    def attend(self, q_extra=None, k_text=None, v_text=None, stream=None):
        adas_sparse_attn_fwd(self.geom, self.q_cube, self.k_cube, self.v_cube, q_extra, k_text, v_text,
                             self.sel_count, self.sel_idx, self.out_raster, self.out_extra, self.ws,
                             stream)

    def forward(self, q_raster, k_raster, v_raster, q_extra=None, k_text=None, v_text=None,
                stream=None):
        """Whole path: partition Q/K/V, mean keys, selection, attention."""
        self.build_kv(k_raster, v_raster, stream)
        if self.has_video:
            self.partition_queries(q_raster, stream)
        self.select(q_extra, stream=stream)
        self.attend(q_extra, k_text, v_text, stream)
        return self.out_raster, self.out_extra

    def decode_step(self, q_extra, stream=None):
        """Selection plus attention for extra rows over an already built cache:
        one adas_decode_step call (Top-p, no video rows, no text keys), else
        the selection and attention calls in turn."""
        if self.has_video or self.n_text_kv or self.topk is not None:
            self.select(q_extra, stream=stream)
            self.attend(q_extra, None, None, stream)
            return self.out_extra
        if getattr(self, "ws_decode", None) is None:
            wsd = adas_workspace_bytes(self.geom, self.dtype, ADAS_WS_DECODE, False, self.n_extra)
            self.ws_decode = torch.empty((max(wsd, 1),), device=self.kbar.device, dtype=torch.uint8)
        adas_decode_step(self.geom, q_extra, self.kbar, self.k_cube, self.v_cube, self.p, self.sel_count,
                         self.sel_idx, self.out_extra, self.ws_decode, stream)
        return self.out_extra


class AdasFFN:
    """Buffers and call sequence for one AdaS-FFN layer on one device.

    Weights are bf16 in the nn.Linear layout (w_gate, w_up [inter][hidden],
    w_down [hidden][inter]); n_text text tokens go through the FFN densely.
    """

    def __init__(self, geom: FfnGeometry, p: float, w_gate: torch.Tensor, w_up: torch.Tensor,
                 w_down: torch.Tensor, n_text: int = 0, device="cuda"):
        load()
        self.geom, self.p, self.n_text = geom, float(p), n_text
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        dev = torch.device(device)
        g = geom
        i32 = dict(device=dev, dtype=torch.int32)
        self.act_count = torch.empty((g.n_cubes,), **i32)
        self.act_off = torch.empty((g.n_cubes + 1,), **i32)
        self.act_rows = torch.empty((g.N,), **i32)
        self.act_mask = torch.empty((g.n_cubes, g.mask_words), **i32)
        self.y = torch.empty((g.N, g.hidden), device=dev, dtype=torch.bfloat16)
        self.y_text = torch.empty((n_text, g.hidden), device=dev, dtype=torch.bfloat16) if n_text else None
        ws = adas_ffn_workspace_bytes(g, n_text)
        self.ws = torch.empty((ws,), device=dev, dtype=torch.uint8)

    def select(self, x: torch.Tensor, stream=None):
        adas_ffn_select(self.geom, x, self.p, self.act_count, self.act_off, self.act_rows, self.act_mask,
                        stream)

    def ffn(self, x: torch.Tensor, x_text: Optional[torch.Tensor] = None, stream=None):
        adas_ffn_fwd(self.geom, x, x_text, self.w_gate, self.w_up, self.w_down, self.act_off,
                     self.act_rows, self.act_mask, self.y, self.y_text, self.ws, stream)

    def forward(self, x: torch.Tensor, x_text: Optional[torch.Tensor] = None, stream=None):
        self.select(x, stream)
        self.ffn(x, x_text, stream)
        return self.y, self.y_text


class StreamingCache:
    """A cube-layout video KV cache allocated for `geom.T` frames (or
    `geom.cache_T`) and filled as frames arrive (``append``).  Decode steps
    (``decode``) select among and attend to the cubes of the completed
    temporal blocks."""

    def __init__(self, geom: Geometry, p: float, device="cuda"):
        load()
        self.cap = geom.cache_T or geom.T
        self.geom = Geometry(self.cap, geom.H, geom.W, geom.ct, geom.ch, geom.cw, geom.n_q_heads,
                             geom.n_kv_heads, geom.head_dim, geom.head_map, self.cap)
        self.p = float(p)
        g = self.geom
        dev = torch.device(device)
        self.device = dev
        bf = dict(device=dev, dtype=torch.bfloat16)
        self.k_cache = torch.empty((g.n_kv_heads, g.NS, g.head_dim), **bf)
        self.v_cache = torch.empty((g.n_kv_heads, g.NS // g.S, g.head_dim, g.S), **bf)
        self.kbar = torch.empty((g.n_kv_heads, g.NS // g.S, g.head_dim), device=dev, dtype=torch.float32)
        self.ksum = torch.empty((adas_cache_sum_bytes(g),), device=dev, dtype=torch.uint8)
        self.frames = 0
        self._bufs = {}

    @property
    def complete_frames(self) -> int:
        return self.frames // self.geom.ct * self.geom.ct

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        """k_new, v_new [n*H*W][Hkv][d] bf16: the next n frames."""
        n = k_new.shape[0] // (self.geom.H * self.geom.W)
        adas_cache_append(self.geom, self.frames, k_new, v_new, self.k_cache, self.v_cache, self.kbar,
                          self.ksum, stream)
        self.frames += n

    def decode_geometry(self) -> Geometry:
        g = self.geom
        return Geometry(self.complete_frames, g.H, g.W, g.ct, g.ch, g.cw, g.n_q_heads, g.n_kv_heads,
                        g.head_dim, g.head_map, self.cap)

    def decode(self, q_extra: torch.Tensor, stream=None):
        """One decode step for q_extra [n][Hq][d] over the completed cubes;
        returns (out [n][Hq][d], sel_count, sel_idx)."""
        if self.complete_frames == 0:
            raise ValueError("no complete temporal block in the cache yet")
        g = self.decode_geometry()
        n = q_extra.shape[0]
        key = (g.T, n)
        if key not in self._bufs:
            cap = adas_sel_capacity(g, False, n)
            ws_s = adas_workspace_bytes(g, torch.bfloat16, ADAS_WS_SELECT, False, n)
            ws_a = adas_workspace_bytes(g, torch.bfloat16, ADAS_WS_ATTN, False, n)
            dev = self.device
            self._bufs[key] = (
                torch.empty((g.n_q_heads, n), device=dev, dtype=torch.int32),
                torch.empty((cap,), device=dev, dtype=torch.int32),
                torch.empty((max(ws_s, 1),), device=dev, dtype=torch.uint8),
                torch.empty((max(ws_a, 1),), device=dev, dtype=torch.uint8),
                torch.empty((n, g.n_q_heads, g.head_dim), device=dev, dtype=torch.bfloat16))
        cnt, idx, ws_s, ws_a, out = self._bufs[key]
        adas_select_topp(g, None, q_extra, self.kbar, self.p, cnt, idx, ws_s, stream)
        adas_sparse_attn_fwd(g, None, self.k_cache, self.v_cache, q_extra, None, None, cnt, idx, None, out,
                             ws_a, stream)
        return out, cnt, idx


class AdasAttentionGrad:
    """Forward with log-sum-exp and backward of the sparse attention for one
    layer (video rows, and extra rows that attend their selected cubes and,
    with n_text_kv = n_extra, the causal text keys of a text prefill): the
    fine-tuning step the AdaSpark pages adapt the backbone with.  The
    selection is computed in the forward and held fixed in the backward.
    The text keys' gradients land in ``dk_text`` / ``dv_text``."""

    def __init__(self, geom: Geometry, p: float, has_video: bool = True, n_extra: int = 0, device="cuda",
                 topk: Optional[int] = None, n_text_kv: int = 0):
        if n_text_kv not in (0, n_extra):
            raise ValueError("n_text_kv must be 0 or n_extra")
        self.fwd = AdasAttention(geom, torch.bfloat16, p, has_video=has_video, n_extra=n_extra,
                                 n_text_kv=n_text_kv, device=device, topk=topk)
        self.n_text_kv = n_text_kv
        self._text = (None, None)
        g = geom
        dev = torch.device(device)
        e = dict(device=dev, dtype=torch.bfloat16)
        self.v_tok = torch.empty((g.n_kv_heads, g.NS, g.head_dim), **e)
        self.k_vt = torch.empty((g.n_kv_heads, g.NS // g.S, g.head_dim, g.S), **e)
        self.lse = torch.empty(tuple(self.fwd.sel_count.shape), device=dev, dtype=torch.float32)
        f = dict(device=dev, dtype=torch.float32)
        self.dq = torch.empty((g.N, g.n_q_heads, g.head_dim), **f) if has_video else None
        self.dq_extra = torch.empty((n_extra, g.n_q_heads, g.head_dim), **f) if n_extra else None
        self.dk = torch.empty((g.N, g.n_kv_heads, g.head_dim), **f)
        self.dv = torch.empty((g.N, g.n_kv_heads, g.head_dim), **f)
        self.dk_text = torch.empty((n_text_kv, g.n_kv_heads, g.head_dim), **f) if n_text_kv else None
        self.dv_text = torch.empty((n_text_kv, g.n_kv_heads, g.head_dim), **f) if n_text_kv else None
        ws = adas_workspace_bytes(g, torch.bfloat16, ADAS_WS_BWD, has_video, n_extra)
        self.ws_bwd = torch.empty((ws,), device=dev, dtype=torch.uint8)

    def forward(self, q_raster, k_raster, v_raster, q_extra=None, stream=None, k_text=None, v_text=None):
        """k_text / v_text [n_text_kv][Hkv][d]: the text prefill's causal text
        keys and values (required when n_text_kv > 0)."""
        L = self.fwd
        if self.n_text_kv and (k_text is None or v_text is None):
            raise ValueError("this layer has causal text keys: pass k_text and v_text")
        self._text = (k_text, v_text) if self.n_text_kv else (None, None)
        L.build_kv(k_raster, v_raster, stream)
        adas_cube_partition(L.geom, v_raster, self.v_tok, None, stream)
        adas_cube_partition(L.geom, k_raster, self.k_vt, None, stream, layout=ADAS_LAYOUT_VT)
        if L.has_video:
            L.partition_queries(q_raster, stream)
        L.select(q_extra, stream=stream)
        adas_sparse_attn_fwd_lse(L.geom, L.q_cube, L.k_cube, L.v_cube, q_extra, self._text[0], self._text[1],
                                 L.sel_count, L.sel_idx, L.out_raster, L.out_extra, self.lse, L.ws, stream)
        return L.out_raster, L.out_extra

    def backward(self, dout_raster, dout_extra=None, q_extra=None, stream=None):
        L = self.fwd
        adas_sparse_attn_bwd(L.geom, L.q_cube, L.k_cube, self.v_tok, self.k_vt, q_extra, L.sel_count, L.sel_idx,
                             L.out_raster, L.out_extra, self.lse, dout_raster, dout_extra, self.dq, self.dq_extra,
                             self.dk, self.dv, self.ws_bwd, stream, k_text=self._text[0], v_text=self._text[1],
                             dk_text=self.dk_text, dv_text=self.dv_text)
        return self.dq, self.dq_extra, self.dk, self.dv

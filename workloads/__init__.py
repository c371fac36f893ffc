"""Seeded synthetic inputs for AdaS-Attn (adaptive cube-selective attention).

This module only *draws* inputs.  It holds none of the method's arithmetic:
no cube numbering, no means, no scores, no selection, no attention.  Both the
CPU oracle (``oracle/``) and the HIP path read the same arrays from here.

Source of the shapes: AdaSpark (CVPR 2026), the papernotes.org summary
("关键设计" items 1-2: h x w x t cubes, Top-p over preceding cubes) and the
thelatestinai.com listing (Table 3: 4x4x4 cubes; Table 5: Qwen2.5-VL-3B/7B
backbones).  The value distributions are the synthetic stand-ins for the
benchmarks the pages evaluate on (MLVU, VideoMME, VideoNIAH, ...), which are
not available here:

* per-cube centre ``c ~ N(0, c_std^2)`` per KV head and per dim,
* keys ``K = c_cube(token) + sigma_cube * N(0,1)``,
* ``Q, V ~ N(0,1)``; text / decode queries and text K/V ``~ N(0,1)``.

Layouts are token-major, as a QKV projection emits them:
``q[N][Hq][d]``, ``k[N][Hkv][d]``, ``v[N][Hkv][d]`` with raster token index
``n = (f*H + y)*W + x``; text tensors ``[Nt][heads][d]``.

bf16 tensors are returned as ``np.uint16`` bit patterns (round-to-nearest-even
from the float32 draw); f32 tensors as ``np.float32``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "generate", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "FfnWorkload", "FFN_WORKLOADS", "get_ffn", "generate_ffn",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic AdaS-Attn layer input.

    ``ct, ch, cw`` are the cube's temporal / height / width extents (the
    pages write the cube as h x w x t).
    """
    name: str
    T: int
    H: int
    W: int
    ct: int
    ch: int
    cw: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    p: float
    seed: int
    c_std: float = 1.0
    noise_std: float = 0.3
    mixed_noise: bool = False  # half the cubes (seeded permutation) get std 1.0
    video_queries: bool = True
    n_text: int = 0            # text queries appended after the video (causal among themselves)
    text_kv: bool = False      # text tokens also carry K/V (prefill with text)
    n_decode: int = 0          # independent decode queries over the video cache
    description: str = ""

    # derived sizes (pure shape bookkeeping)
    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def cube_size(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def n_cubes(self) -> int:
        return self.n_tokens // self.cube_size

    @property
    def n_extra_queries(self) -> int:
        """Rows that are not video rows: text queries or decode queries."""
        return self.n_text + self.n_decode

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(**kw) -> Workload:
    return Workload(**kw)


# The five synthetic configurations (sizes from the AdaSpark listing's
# backbones and cube ablations; seeds 1000 + k).
WORKLOADS = {
    # Tiny fp32 case, cube h x w x t = 4x4x2 -> 16 cubes of 32 tokens.
    "tiny": _w(name="tiny", T=8, H=8, W=8, ct=2, ch=4, cw=4, n_q_heads=1,
               n_kv_heads=1, head_dim=64, dtype="f32", p=0.7, seed=1001,
               description="Tiny: 1 head, d=64, fp32, 8x8x8 grid, cube 4x4x2 (16 cubes of 32), p=0.7"),
    # The same tiny grid read as '32 cubes of 16': cube h x w x t = 2x2x4.
    "tiny_b": _w(name="tiny_b", T=8, H=8, W=8, ct=4, ch=2, cw=2, n_q_heads=1,
                 n_kv_heads=1, head_dim=64, dtype="f32", p=0.7, seed=1001,
                 description="Tiny, alternative reading: cube 2x2x4 (32 cubes of 16), p=0.7"),
    "qwen3b": _w(name="qwen3b", T=64, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=16,
                 n_kv_heads=2, head_dim=128, dtype="bf16", p=0.7, seed=1002, c_std=1.5,
                 description="Qwen2.5-VL-3B-shaped layer: 16/2 heads, d=128, bf16, 64x16x16 grid, cube 4x4x4 (256 cubes of 64), p=0.7"),
    "qwen7b": _w(name="qwen7b", T=256, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=28,
                 n_kv_heads=4, head_dim=128, dtype="bf16", p=0.7, seed=1003,
                 mixed_noise=True,
                 description="Qwen2.5-VL-7B-shaped layer: 28/4 heads, d=128, bf16, 256x16x16 grid, cube 4x4x4 (1024 cubes), mixed key noise 0.3/1.0"),
    "hour": _w(name="hour", T=512, H=16, W=16, ct=2, ch=8, cw=8, n_q_heads=28,
               n_kv_heads=4, head_dim=128, dtype="bf16", p=0.9, seed=1004,
               n_text=256, text_kv=True,
               description="Hour-scale prefill: 28/4 heads, d=128, bf16, 512x16x16 grid, cube 8x8x2 (1024 cubes of 128), p=0.9, +256 causal text queries"),
    "decode": _w(name="decode", T=1024, H=16, W=16, ct=4, ch=4, cw=4, n_q_heads=28,
                 n_kv_heads=4, head_dim=128, dtype="bf16", p=0.7, seed=1005,
                 video_queries=False, n_decode=64,
                 description="Decode-shaped: 64 independent query tokens over a 1024x16x16 KV cache, 28/4 heads, cube 4x4x4 (4096 cubes), p=0.7"),
}
for _p in (0.5, 0.7, 0.9):
    _name = f"qwen7b_p{int(round(_p * 10)):02d}"
    WORKLOADS[_name] = WORKLOADS["qwen7b"].replace(name=_name, p=_p)


def get(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return wl.replace(**overrides) if overrides else wl


# --------------------------------------------------------------------------
# bf16 bit conversions (data representation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def _expand_cubes(a: np.ndarray, wl: Workload) -> np.ndarray:
    """Broadcast a per-cube array shaped (nT, nH, nW, ...) to every token,
    giving (T*H*W, ...) in raster order, with np.repeat along each grid axis."""
    a = np.repeat(a, wl.ct, axis=0)
    a = np.repeat(a, wl.ch, axis=1)
    a = np.repeat(a, wl.cw, axis=2)
    return a.reshape((wl.n_tokens,) + a.shape[3:])


def generate(wl: Workload) -> dict:
    """Draw every input tensor of ``wl``.

    Draw order from ``np.random.Generator(PCG64(seed))`` (all float32 standard
    normals): cube centres ``(Hkv, nT, nH, nW, d)``; for mixed noise a
    permutation of the cube slots; key noise ``(N, Hkv, d)``; video queries
    ``(N, Hq, d)`` when present; values ``(N, Hkv, d)``; then text queries
    ``(Nt, Hq, d)`` and, with text K/V, text keys and values
    ``(Nt, Hkv, d)``; or decode queries ``(Nd, Hq, d)``.
    """
    if wl.T % wl.ct or wl.H % wl.ch or wl.W % wl.cw:
        raise ValueError("cube extents must divide the grid")
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    nT, nH, nW = wl.T // wl.ct, wl.H // wl.ch, wl.W // wl.cw
    N, Hq, Hkv, d = wl.n_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim

    centres = rng.standard_normal((Hkv, nT, nH, nW, d), dtype=np.float32) * np.float32(wl.c_std)
    sigma = np.full((nT, nH, nW), wl.noise_std, dtype=np.float32)
    if wl.mixed_noise:
        order = rng.permutation(nT * nH * nW)
        flat = sigma.reshape(-1)
        flat[order[: (nT * nH * nW) // 2]] = 1.0
    noise = rng.standard_normal((N, Hkv, d), dtype=np.float32)
    centre_tok = _expand_cubes(np.moveaxis(centres, 0, 3), wl)        # (N, Hkv, d)
    sigma_tok = _expand_cubes(sigma, wl)                               # (N,)
    k32 = centre_tok + sigma_tok[:, None, None] * noise
    del noise, centre_tok

    out = {"workload": wl}
    if wl.video_queries:
        out["q"] = _cast(rng.standard_normal((N, Hq, d), dtype=np.float32), wl.dtype)
    out["k"] = _cast(k32, wl.dtype)
    del k32
    out["v"] = _cast(rng.standard_normal((N, Hkv, d), dtype=np.float32), wl.dtype)
    if wl.n_text:
        out["q_text"] = _cast(rng.standard_normal((wl.n_text, Hq, d), dtype=np.float32), wl.dtype)
        if wl.text_kv:
            out["k_text"] = _cast(rng.standard_normal((wl.n_text, Hkv, d), dtype=np.float32), wl.dtype)
            out["v_text"] = _cast(rng.standard_normal((wl.n_text, Hkv, d), dtype=np.float32), wl.dtype)
    if wl.n_decode:
        out["q_text"] = _cast(rng.standard_normal((wl.n_decode, Hq, d), dtype=np.float32), wl.dtype)
    return out


# --------------------------------------------------------------------------
# AdaS-FFN inputs (the papernotes.org page, key design 3: tokens of each cube
# are kept or skipped by their L2 norm; the thelatestinai.com listing, Table 5:
# Qwen2.5-VL-3B / 7B backbones, whose MLP is SwiGLU)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class FfnWorkload:
    """One synthetic AdaS-FFN layer input.

    Video hidden states ``x[N][hidden]`` in raster token order on a T x H x W
    grid cut into ct x ch x cw cubes, optional text hidden states
    ``x_text[Nt][hidden]``, and SwiGLU weights in the nn.Linear layout:
    ``w_gate, w_up [inter][hidden]``, ``w_down [hidden][inter]``.

    Token magnitudes vary so that the norm-based selection has something to
    adapt to: token n is ``exp(s_c * z_n) * u_n`` with ``u_n ~ N(0, I)``,
    ``z_n ~ N(0, 1)`` and ``s_c`` = ``spread_hi`` for a seeded half of the
    cubes ("busy" cubes, a few dominant tokens) and ``spread_lo`` for the rest
    ("flat" cubes, near-uniform norms).
    """
    name: str
    T: int
    H: int
    W: int
    ct: int
    ch: int
    cw: int
    hidden: int
    inter: int
    p: float
    seed: int
    n_text: int = 0
    spread_lo: float = 0.2
    spread_hi: float = 1.0
    description: str = ""

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def cube_size(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def n_cubes(self) -> int:
        return self.n_tokens // self.cube_size

    def replace(self, **kw) -> "FfnWorkload":
        return dataclasses.replace(self, **kw)


FFN_WORKLOADS = {
    "ffn_tiny": FfnWorkload(name="ffn_tiny", T=4, H=8, W=8, ct=2, ch=4, cw=4, hidden=256, inter=384,
                            p=0.7, seed=2001, n_text=5,
                            description="Tiny AdaS-FFN: 4x8x8 grid, cube 4x4x2 (8 cubes of 32), hidden 256, "
                                        "inter 384, 5 text tokens, p=0.7"),
    "ffn3b": FfnWorkload(name="ffn3b", T=64, H=16, W=16, ct=4, ch=4, cw=4, hidden=2048, inter=11008,
                         p=0.7, seed=2002,
                         description="Qwen2.5-VL-3B-shaped FFN: 64x16x16 grid, cube 4x4x4 (256 cubes of 64), "
                                     "hidden 2048, inter 11008, p=0.7"),
    "ffn7b": FfnWorkload(name="ffn7b", T=256, H=16, W=16, ct=4, ch=4, cw=4, hidden=3584, inter=18944,
                         p=0.7, seed=2003,
                         description="Qwen2.5-VL-7B-shaped FFN: 256x16x16 grid, cube 4x4x4 (1024 cubes of 64), "
                                     "hidden 3584, inter 18944, p=0.7"),
    "ffn_hour": FfnWorkload(name="ffn_hour", T=512, H=16, W=16, ct=2, ch=8, cw=8, hidden=3584, inter=18944,
                            p=0.9, seed=2004, n_text=256,
                            description="Hour-scale FFN: 512x16x16 grid, cube 8x8x2 (1024 cubes of 128), "
                                        "hidden 3584, inter 18944, p=0.9, +256 text tokens"),
}


def get_ffn(name: str, **overrides) -> FfnWorkload:
    wl = FFN_WORKLOADS[name]
    return wl.replace(**overrides) if overrides else wl


def generate_ffn(wl: FfnWorkload) -> dict:
    """Draw every input of ``wl`` as bf16 bits.

    Draw order from ``np.random.Generator(PCG64(seed))``: a permutation of the
    cube slots (its first half are the busy cubes); per-token log-magnitudes
    ``z (N,)``; directions ``u (N, hidden)``; text states ``(Nt, hidden)``;
    ``w_gate``, ``w_up`` ``(inter, hidden)`` scaled by 1/sqrt(hidden);
    ``w_down`` ``(hidden, inter)`` scaled by 1/sqrt(inter).  All float32
    standard normals, rounded to bf16 (RNE).
    """
    if wl.T % wl.ct or wl.H % wl.ch or wl.W % wl.cw:
        raise ValueError("cube extents must divide the grid")
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    nT, nH, nW = wl.T // wl.ct, wl.H // wl.ch, wl.W // wl.cw
    N, Hd, I = wl.n_tokens, wl.hidden, wl.inter
    order = rng.permutation(nT * nH * nW)
    spread = np.full(nT * nH * nW, wl.spread_lo, dtype=np.float32)
    spread[order[: (nT * nH * nW) // 2]] = wl.spread_hi
    spread_tok = _expand_cubes(spread.reshape(nT, nH, nW), wl)          # (N,)
    z = rng.standard_normal(N, dtype=np.float32)
    mag = np.exp(spread_tok * z).astype(np.float32)
    out = {"workload": wl}
    u = rng.standard_normal((N, Hd), dtype=np.float32)
    u *= mag[:, None]
    out["x"] = f32_to_bf16_bits(u)
    del u
    out["x_text"] = f32_to_bf16_bits(rng.standard_normal((wl.n_text, Hd), dtype=np.float32))
    for name, shape, fan_in in (("w_gate", (I, Hd), Hd), ("w_up", (I, Hd), Hd), ("w_down", (Hd, I), I)):
        w = rng.standard_normal(shape, dtype=np.float32)
        w *= np.float32(1.0 / np.sqrt(fan_in))
        out[name] = f32_to_bf16_bits(w)
        del w
    return out

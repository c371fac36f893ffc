"""GPU cube partition in both layouts against the oracle's partition, bit for
bit, through the C ABI (adas_cube_partition).

ADAS_LAYOUT_TOKENS must equal the oracle's cube-contiguous copy and perm;
ADAS_LAYOUT_VT must equal that copy transposed per cube with the column
permutation include/adas.h states (bits 2 and 3 swapped inside complete aligned
groups of 16 offsets).  The shapes cover 16-byte stores of 8 bf16 or 4 float32
positions (S = 24, 32, 64, 128; S = 24 ends in a partial group of 8), the
element-wise path for an S that is not a multiple of the vector width (S = 9),
and a head count other than the attention's.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import adas_oracle as O
from tests.gpu_harness import bits, log, to_vt

pytestmark = pytest.mark.gpu

SHAPES = [
    # T, H, W, ct, ch, cw, dtype, d, heads
    (4, 16, 16, 4, 4, 4, "bf16", 128, 2),
    (8, 16, 16, 2, 8, 8, "bf16", 128, 3),
    (4, 8, 8, 2, 4, 4, "f32", 64, 1),
    (2, 12, 12, 2, 3, 4, "bf16", 128, 2),
    (4, 6, 6, 1, 3, 3, "bf16", 64, 2),
    (8, 16, 16, 2, 8, 8, "f32", 64, 2),
    (2, 8, 8, 1, 2, 2, "f32", 128, 1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:6])) + f"_{s[6]}_d{s[7]}_h{s[8]}")
def test_partition_layouts_bit_exact(shape):
    from adaptive_cube_sparse_amd import ADAS_LAYOUT_VT, Geometry, adas_cube_partition
    T, H, W, ct, ch, cw, dt, d, nh = shape
    N, S = T * H * W, ct * ch * cw
    log(f"[partition] grid {T}x{H}x{W} cube ({ct},{ch},{cw}) S {S} {dt} d {d} heads {nh}")
    rng = np.random.default_rng(S * 1000 + d + nh)
    if dt == "bf16":
        raw = rng.integers(0, 1 << 16, size=(N, nh, d), dtype=np.uint16)
        x = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    else:
        raw = rng.integers(0, 1 << 32, size=(N, nh, d), dtype=np.uint32)
        x = torch.from_numpy(raw.view(np.int32)).view(torch.float32).to("cuda:0")
    geom = Geometry(T, H, W, ct, ch, cw, nh, nh, d)
    tok = torch.empty((nh, N, d), dtype=x.dtype, device=x.device)
    vt = torch.empty((nh, N // S, d, S), dtype=x.dtype, device=x.device)
    perm = torch.empty((N,), dtype=torch.int32, device=x.device)
    adas_cube_partition(geom, x, tok, perm)
    adas_cube_partition(geom, x, vt, None, layout=ADAS_LAYOUT_VT)
    torch.cuda.synchronize()
    g = O.Geometry(T, H, W, ct, ch, cw)
    want, want_perm = O.partition(raw, g)
    got_tok = bits(tok) if dt == "bf16" else tok.cpu().view(torch.int32).numpy().view(np.uint32)
    got_vt = bits(vt) if dt == "bf16" else vt.cpu().view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(perm.cpu().numpy(), want_perm), "perm differs"
    assert np.array_equal(got_tok, want), "token layout differs"
    assert np.array_equal(got_vt, to_vt(want, S)), "VT layout differs"


KEY_SHAPES = [
    # T, H, W, ct, ch, cw, dtype, d, kv heads, value scale spread (binades)
    (4, 16, 16, 4, 4, 4, "bf16", 128, 2, 0),
    (8, 16, 16, 2, 8, 8, "bf16", 128, 3, 0),
    (4, 16, 16, 4, 8, 8, "bf16", 64, 2, 36),     # S = 256, magnitudes over 2^37
    (2, 12, 12, 2, 3, 4, "bf16", 128, 1, 0),     # S = 24
    (4, 6, 6, 1, 3, 3, "bf16", 64, 2, 0),        # S = 9
    (4, 16, 16, 4, 8, 8, "f32", 64, 2, 20),      # float32 keys over 2^21
    (2, 8, 8, 1, 2, 2, "f32", 128, 1, 0),
    (8, 16, 16, 8, 8, 8, "bf16", 128, 1, 0),     # S = 512
]


@pytest.mark.parametrize("shape", KEY_SHAPES,
                         ids=lambda s: "x".join(map(str, s[:6])) + f"_{s[6]}_d{s[7]}_h{s[8]}_e{s[9]}")
def test_partition_keys_one_pass(shape):
    """adas_cube_partition_keys: k_cube and perm bit-equal to the oracle's
    partition, kbar bit-equal to the oracle's float64 means rounded once (and
    to adas_cube_mean_keys).  Keys are N(0,1), or, with a spread e, a random
    sign times [1, 2) times 2^u, u uniform in 0..e: magnitudes within a
    factor 2^(e+1), the widest range include/adas.h promises agreement for."""
    from adaptive_cube_sparse_amd import Geometry, adas_cube_mean_keys, adas_cube_partition_keys
    T, H, W, ct, ch, cw, dt, d, nh, spread = shape
    N, S = T * H * W, ct * ch * cw
    log(f"[partition_keys] grid {T}x{H}x{W} cube ({ct},{ch},{cw}) S {S} {dt} d {d} kv heads {nh} "
        f"spread 2^{spread}")
    rng = np.random.default_rng(7 * S + d + nh + spread)
    if spread:
        x32 = (rng.choice([-1.0, 1.0], size=(N, nh, d)) * (1.0 + rng.random((N, nh, d)))
               * np.exp2(rng.integers(0, spread + 1, size=(N, nh, d)))).astype(np.float32)
    else:
        x32 = rng.standard_normal((N, nh, d)).astype(np.float32)
    if dt == "bf16":
        raw = workloads.f32_to_bf16_bits(x32)
        x = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    else:
        raw = x32
        x = torch.from_numpy(raw).to("cuda:0")
    geom = Geometry(T, H, W, ct, ch, cw, nh, nh, d)
    kc = torch.empty((nh, N, d), dtype=x.dtype, device=x.device)
    perm = torch.empty((N,), dtype=torch.int32, device=x.device)
    kbar = torch.empty((nh, N // S, d), dtype=torch.float32, device=x.device)
    kbar2 = torch.empty_like(kbar)
    adas_cube_partition_keys(geom, x, kc, perm, kbar)
    adas_cube_mean_keys(geom, kc, kbar2)
    torch.cuda.synchronize()
    g = O.Geometry(T, H, W, ct, ch, cw)
    want, want_perm = O.partition(raw, g)
    got = bits(kc) if dt == "bf16" else kc.cpu().numpy()
    assert np.array_equal(perm.cpu().numpy(), want_perm), "perm differs"
    assert np.array_equal(got.view(np.uint16 if dt == "bf16" else np.uint32),
                          want.view(np.uint16 if dt == "bf16" else np.uint32)), "k_cube differs"
    want_kb = O.kbar_to_f32(O.mean_keys(want, g)).view(np.uint32)
    kb = kbar.cpu().numpy().view(np.uint32)
    assert np.array_equal(kb, want_kb), f"kbar differs from the oracle in {int((kb != want_kb).sum())} entries"
    assert np.array_equal(kb, kbar2.cpu().numpy().view(np.uint32)), "kbar differs from adas_cube_mean_keys"

"""Pins for the oracle's cube partition (O1) and mean keys (O2).

AdaSpark, papernotes.org, key design 1 (h x w x t cube partition, the cube is
the atomic unit) and key design 2 (the mean key kbar_j of each cube).
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import adas_oracle as O
from tests.conftest import GOLDEN

GEOMS = [
    O.Geometry(2, 4, 4, 1, 2, 2),
    O.Geometry(8, 8, 8, 2, 4, 4),      # tiny, cube 4x4x2
    O.Geometry(8, 8, 8, 4, 2, 2),      # tiny, cube 2x2x4
    O.Geometry(6, 6, 10, 3, 2, 5),     # non-square, non power-of-two cube
    O.Geometry(4, 16, 16, 2, 8, 8),    # 'hour'-style 8x8x2 cube
]


def brute_force_cube_tokens(g: O.Geometry):
    """Enumerate each cube's tokens with nested loops over cube blocks and
    in-cube offsets; independent of the oracle's closed form."""
    cubes = []
    for bf in range(g.nT):
        for by in range(g.nH):
            for bx in range(g.nW):
                toks = []
                for dt in range(g.ct):
                    for dy in range(g.ch):
                        for dx in range(g.cw):
                            f, y, x = bf * g.ct + dt, by * g.ch + dy, bx * g.cw + dx
                            toks.append((f * g.H + y) * g.W + x)
                cubes.append(toks)
    return cubes


def test_partition_golden():
    gold = json.load(open(os.path.join(GOLDEN, "partition_2x4x4.json")))
    g = O.Geometry(gold["T"], gold["H"], gold["W"], gold["ct"], gold["ch"], gold["cw"])
    x = np.arange(g.N, dtype=np.int64).reshape(g.N, 1, 1)
    x_cube, perm = O.partition(x, g)
    got = perm.reshape(g.n_cubes, g.S).tolist()
    assert got == gold["cube_tokens"]
    assert x_cube[0, :, 0].tolist() == perm.tolist()


@pytest.mark.parametrize("g", GEOMS, ids=lambda g: f"{g.T}x{g.H}x{g.W}_c{g.ct}{g.ch}{g.cw}")
def test_partition_matches_brute_force_and_is_bijection(g):
    _, perm = O.partition(np.zeros((g.N, 1, 1), np.float32), g)
    assert sorted(perm.tolist()) == list(range(g.N))
    assert perm.reshape(g.n_cubes, g.S).tolist() == brute_force_cube_tokens(g)


@pytest.mark.parametrize("g", GEOMS, ids=lambda g: f"{g.T}x{g.H}x{g.W}_c{g.ct}{g.ch}{g.cw}")
def test_partition_round_trip_and_head_major(g):
    rng = np.random.default_rng(7)
    x = rng.integers(0, 2**16, size=(g.N, 3, 5), dtype=np.uint16)
    x_cube, perm = O.partition(x, g)
    assert x_cube.shape == (3, g.N, 5) and x_cube.dtype == np.uint16
    back = np.empty_like(x)
    back[perm] = np.swapaxes(x_cube, 0, 1)
    np.testing.assert_array_equal(back, x)


def test_cubes_are_spatiotemporal_boxes():
    g = O.Geometry(8, 8, 8, 2, 4, 4)
    _, perm = O.partition(np.zeros((g.N, 1, 1), np.float32), g)
    for c in range(g.n_cubes):
        toks = perm[c * g.S:(c + 1) * g.S]
        f, y, x = toks // 64, (toks // 8) % 8, toks % 8
        assert (f.max() - f.min() + 1, y.max() - y.min() + 1, x.max() - x.min() + 1) == (2, 4, 4)
        assert len(set(zip(f, y, x))) == g.S
    first = [perm[c * g.S] for c in range(g.n_cubes)]
    assert first == sorted(first), "cubes are ordered by their first raster token"


def test_rejects_non_dividing_cube():
    with pytest.raises(ValueError):
        O.Geometry(8, 8, 8, 3, 4, 4)


def _brute_force_means(k_raster_f64, g):
    """Average each cube's keys straight from raster order with explicit loops."""
    N, Hkv, d = k_raster_f64.shape
    out = np.zeros((Hkv, g.n_cubes, d))
    for ci, toks in enumerate(brute_force_cube_tokens(g)):
        acc = np.zeros((Hkv, d))
        for n in toks:
            acc += k_raster_f64[n]
        out[:, ci] = acc / len(toks)
    return out


@pytest.mark.parametrize("name", ["tiny", "tiny_b"])
def test_mean_keys_match_brute_force(name):
    wl = workloads.get(name)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    k_cube, _ = O.partition(data["k"], g)
    kbar = O.mean_keys(k_cube, g)
    ref = _brute_force_means(O.to_f64(data["k"]), g)
    np.testing.assert_allclose(kbar, ref, rtol=0, atol=1e-13)


def test_mean_keys_bf16_gqa_brute_force():
    wl = workloads.Workload(name="t", T=4, H=8, W=8, ct=2, ch=4, cw=4, n_q_heads=4,
                            n_kv_heads=2, head_dim=16, dtype="bf16", p=0.7, seed=5)
    data = workloads.generate(wl)
    g = O.Geometry.of(wl)
    k_cube, _ = O.partition(data["k"], g)
    np.testing.assert_allclose(O.mean_keys(k_cube, g), _brute_force_means(O.to_f64(data["k"]), g),
                               rtol=0, atol=1e-13)


def test_mean_of_identical_keys_is_the_key():
    g = O.Geometry(4, 4, 4, 2, 2, 2)
    rng = np.random.default_rng(3)
    per_cube = rng.standard_normal((2, g.n_cubes, 8)).astype(np.float32)
    k_cube = np.repeat(per_cube, g.S, axis=1)              # every token of cube j = per_cube[j]
    np.testing.assert_array_equal(O.mean_keys(k_cube, g), per_cube.astype(np.float64))


def test_mean_keys_exact_for_bf16_power_of_two_cubes():
    """For bf16 keys and S = 2^k the float64 sum is exact, so the float64 mean
    equals the rational mean and its float32 rounding is unique."""
    g = O.Geometry(4, 8, 8, 4, 4, 4)  # S = 64
    rng = np.random.default_rng(11)
    k = workloads.f32_to_bf16_bits(rng.standard_normal((1, g.N, 4)).astype(np.float32))
    kbar = O.mean_keys(k, g)
    vals = O.to_f64(k)
    for j in range(g.n_cubes):
        for dd in range(4):
            exact = sum(Fraction(float(v)) for v in vals[0, j * g.S:(j + 1) * g.S, dd]) / g.S
            assert Fraction(float(kbar[0, j, dd])) == exact
            assert O.kbar_to_f32(kbar)[0, j, dd] == np.float32(float(exact))


def test_mean_keys_linear_in_keys():
    g = O.Geometry(4, 4, 4, 2, 2, 2)
    rng = np.random.default_rng(4)
    a = rng.standard_normal((1, g.N, 3))
    b = rng.standard_normal((1, g.N, 3))
    np.testing.assert_allclose(O.mean_keys(2 * a - b, g), 2 * O.mean_keys(a, g) - O.mean_keys(b, g),
                               atol=1e-13)

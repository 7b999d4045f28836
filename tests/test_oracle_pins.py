"""Pins for the fp64 CPU oracle: each test checks it against something other
than itself (a library routine, a closed form, a hand-computed case, an
invariant, or the independent numpy brute force)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(x):
    return (bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def _rand(shape, seed, dtype="f32"):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _sdpa(q, k, v, scale=None):
    """Library dense attention in float64 on the CPU."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale).numpy()


def _coords_tiles(grid, tile):
    """Tile id of each token from coordinates (used by the probe tests)."""
    T, H, W = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    ny, nx = -(-H // tile[1]), -(-W // tile[2])
    return ((t // tile[0]) * ny + y // tile[1]) * nx + x // tile[2]


RAGGED = [((3, 10, 12), (1, 4, 8)), ((2, 5, 7), (2, 2, 3)), ((4, 8, 8), (1, 4, 4))]


@pytest.mark.parametrize("grid,tile", RAGGED)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ones_mask_is_dense_attention(oracle_lib, grid, tile, dtype):
    heads, d = 2, 16
    N = int(np.prod(grid))
    q, k, v = (_rand((heads, N, d), s, dtype) for s in (1, 2, 3))
    nT = oracle.num_tiles(grid, tile)
    M = np.ones((heads, nT, nT), np.uint8)
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)
    ref = _sdpa(_f64(q), _f64(k), _f64(v))
    assert np.abs(O - ref).max() < 1e-12


def test_all_ones_mask_with_explicit_scale(oracle_lib):
    grid, tile = (2, 4, 6), (1, 2, 3)
    q, k, v = (_rand((1, 48, 8), s) for s in (4, 5, 6))
    M = np.ones((1, 8, 8), np.uint8)
    O = oracle.attention(grid, tile, q, k, v, M, scale=0.37, threads=2)
    assert np.abs(O - _sdpa(_f64(q), _f64(k), _f64(v), scale=0.37)).max() < 1e-12


def test_block_diagonal_mask_is_per_tile_attention(oracle_lib):
    # A query whose row keeps only its own tile attends only there: the result
    # equals dense attention inside each tile separately.
    grid, tile = (2, 8, 8), (1, 4, 4)
    T, H, W = grid
    heads, d = 2, 8
    q, k, v = (_rand((heads, T * H * W, d), s) for s in (7, 8, 9))
    nT = oracle.num_tiles(grid, tile)
    M = np.broadcast_to(np.eye(nT, dtype=np.uint8), (heads, nT, nT)).copy()
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)

    def tiles(x):  # [heads, N, d] -> [heads, nT, B, d] via reshapes only
        x = x.reshape(heads, T, H // 4, 4, W // 4, 4, d).transpose(0, 1, 2, 4, 3, 5, 6)
        return x.reshape(heads, nT, 16, d)

    ref = _sdpa(tiles(_f64(q)), tiles(_f64(k)), tiles(_f64(v)))
    got = tiles(O)
    assert np.abs(got - ref).max() < 1e-12


def _random_mask(heads, nT, seed, p=0.4, empty_rows=True):
    rng = np.random.default_rng(seed)
    M = (rng.random((heads, nT, nT)) < p).astype(np.uint8)
    if empty_rows:
        M[0, 0, :] = 0
    return M


@pytest.mark.parametrize("grid,tile", RAGGED)
def test_zero_queries_average_the_kept_values(oracle_lib, grid, tile):
    # q = 0 makes every kept score equal, so each output is the plain mean of
    # the values of the kept keys; an empty row gives 0.
    heads, d = 2, 8
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    q = np.zeros((heads, N, d), np.float32)
    k, v = _rand((heads, N, d), 11), _rand((heads, N, d), 12)
    M = _random_mask(heads, nT, 13)
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)
    tid = _coords_tiles(grid, tile).reshape(-1)
    for h in range(heads):
        for n in range(N):
            kept = M[h, tid[n], tid] != 0
            want = v[h][kept].astype(np.float64).mean(axis=0) if kept.any() else np.zeros(d)
            assert np.abs(O[h, n] - want).max() < 1e-12


def test_constant_values_give_the_constant(oracle_lib):
    grid, tile = (3, 10, 12), (1, 4, 8)
    heads, d, N = 2, 8, 360
    q, k = _rand((heads, N, d), 21), _rand((heads, N, d), 22)
    v = np.full((heads, N, d), 2.5, np.float32)
    M = _random_mask(heads, oracle.num_tiles(grid, tile), 23, empty_rows=False)
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)
    assert np.abs(O - 2.5).max() < 1e-13


def test_tile_indicator_values_give_tile_mass(oracle_lib):
    # v[m, tau] = 1 iff token m lies in tile tau: output column tau is the
    # attention mass on tile tau, exactly 0 for dropped tiles, positive for
    # kept ones, summing to 1.
    grid, tile = (4, 8, 8), (1, 4, 4)
    heads, N = 2, 256
    nT = oracle.num_tiles(grid, tile)
    d = nT
    q, k = _rand((heads, N, d), 31), _rand((heads, N, d), 32)
    tid = _coords_tiles(grid, tile).reshape(-1)
    v = np.zeros((heads, N, d), np.float32)
    v[:, np.arange(N), tid] = 1.0
    M = _random_mask(heads, nT, 33, p=0.5, empty_rows=False)
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)
    for h in range(heads):
        keep = M[h][tid] != 0  # [N, nT]
        assert np.all(O[h][~keep] == 0.0)
        assert np.all(O[h][keep] > 0.0)
        assert np.abs(O[h].sum(axis=1) - 1.0).max() < 1e-13


def test_hand_case(oracle_lib):
    with open(os.path.join(GOLDEN, "hand_case_d1.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], np.float32)[None]
    k = np.array(g["k"], np.float32)[None]
    v = np.array(g["v"], np.float32)[None]
    M = np.array(g["mask"], np.uint8)[None]
    O = oracle.attention(g["grid"], g["tile"], q, k, v, M, scale=g["scale"], threads=1)
    assert abs(O[0, 0, 0] - g["expected_out_row0"]) < g["tolerance"]
    assert abs(O[0, 1, 0] - g["expected_out_row1"]) < g["tolerance"]
    P = oracle.probabilities(g["grid"], g["tile"], q[0], k[0], M[0], scale=g["scale"])
    assert np.abs(P[0] - np.array(g["expected_weights_row0"])).max() < g["tolerance"]


@pytest.mark.parametrize("grid,tile", RAGGED + [((1, 1, 5), (1, 1, 8)), ((5, 3, 3), (2, 3, 3))])
def test_matches_numpy_brute_force(oracle_lib, grid, tile):
    heads, d = 3, 8
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    q, k, v = (_rand((heads, N, d), s, "bf16") for s in (41, 42, 43))
    M = _random_mask(heads, nT, 44, p=0.3)  # asymmetric, with an empty row
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)
    ref = brute.attention(grid, tile, _f64(q), _f64(k), _f64(v), M)
    assert np.abs(O - ref).max() < 1e-12


def test_tiny_workload_matches_brute_force(oracle_lib):
    wl = make_workload("tiny")
    M = oracle.mask_of(wl)
    O = oracle.attention(wl.grid, wl.tile, wl.q, wl.k, wl.v, M, threads=2)
    ref = brute.attention(wl.grid, wl.tile, _f64(wl.q), _f64(wl.k), _f64(wl.v), M)
    assert np.abs(O - ref).max() < 1e-12


def test_small_workload_rows_match_brute_force(oracle_lib):
    wl = make_workload("small", heads=1)
    M = oracle.mask_of(wl)
    rows = np.arange(0, 9600, 37)
    O = oracle.attention_rows(wl.grid, wl.tile, wl.q, wl.k, wl.v, M, rows)
    keep = brute.token_mask(wl.grid, wl.tile, M[0])
    q, k, v = _f64(wl.q[0]), _f64(wl.k[0]), _f64(wl.v[0])
    for c, n in enumerate(rows):
        s = (k[keep[n]] @ q[n]) / np.sqrt(128)
        w = np.exp(s - s.max())
        assert np.abs(O[c] - (w @ v[keep[n]]) / w.sum()).max() < 1e-12


def test_shuffling_keys_inside_a_tile_changes_nothing(oracle_lib):
    grid, tile = (3, 10, 12), (1, 4, 8)
    heads, d, N = 2, 8, 360
    q, k, v = (_rand((heads, N, d), s) for s in (51, 52, 53))
    M = _random_mask(heads, oracle.num_tiles(grid, tile), 54)
    O = oracle.attention(grid, tile, q, k, v, M, threads=2)
    tid = _coords_tiles(grid, tile).reshape(-1)
    rng = np.random.default_rng(55)
    perm = np.arange(N)
    for t in np.unique(tid):
        idx = np.nonzero(tid == t)[0]
        perm[idx] = rng.permutation(idx)
    O2 = oracle.attention(grid, tile, q, k[:, perm], v[:, perm], M, threads=2)
    assert np.abs(O - O2).max() < 1e-13


def test_probabilities_rows_are_distributions(oracle_lib):
    grid, tile = (2, 5, 7), (2, 2, 3)
    N, d = 70, 8
    q, k, v = (_rand((1, N, d), s) for s in (61, 62, 63))
    M = _random_mask(1, oracle.num_tiles(grid, tile), 64)
    P = oracle.probabilities(grid, tile, q[0], k[0], M[0])
    keep = brute.token_mask(grid, tile, M[0])
    assert np.all(P[~keep] == 0.0)
    sums = P.sum(axis=1)
    has = keep.any(axis=1)
    assert np.abs(sums[has] - 1.0).max() < 1e-13 and np.all(sums[~has] == 0.0)
    O = oracle.attention(grid, tile, q, k, v, M, threads=1)
    assert np.abs(P @ v[0].astype(np.float64) - O[0]).max() < 1e-13

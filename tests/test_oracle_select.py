"""Pins of the oracle's tile selection (mean-pooled block scores, per-head
top-k, ties to the lower key tile; SCOPE review page: block-level proxy
scores and per-head Top-k; AdaSpa page: blockified pattern).

Each case fixes the answer independently of the oracle's code: closed-form
scores built into the inputs, the all-tie case, the k = 0 / k = nT ends, and
tile means checked by enumerating tokens with the raster formulas."""

import numpy as np
import pytest

import oracle
from workloads import make_workload


def _tile_of(grid, tile, n):
    T, H, W = grid
    tt, th, tw = tile
    ny, nx = -(-H // th), -(-W // tw)
    t, y, x = n // (H * W), (n // W) % H, n % W
    return ((t // tt) * ny + y // th) * nx + x // tw


@pytest.mark.parametrize("grid,tile", [((3, 10, 12), (1, 4, 8)), ((2, 8, 8), (2, 4, 4))])
def test_tile_means_by_enumeration(grid, tile):
    N = int(np.prod(grid))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((N, 5)).astype(np.float32)
    nT = oracle.num_tiles(grid, tile)
    want = np.zeros((nT, 5))
    cnt = np.zeros(nT)
    for n in range(N):
        t = _tile_of(grid, tile, n)
        want[t] += x[n]
        cnt[t] += 1
    want /= cnt[:, None]
    assert np.allclose(oracle.tile_means(grid, tile, x), want, rtol=0, atol=1e-12)


GRID, TILE = (2, 12, 16), (1, 4, 8)  # tile grid 2 x 3 x 2 = 12 tiles


def _ordered_inputs(sign):
    """K tokens of tile j all equal (j + 1) e_0, Q tokens all sign * e_0:
    score(i, j) = sign (j + 1) / sqrt(d) for every query tile i."""
    N, d = int(np.prod(GRID)), 8
    q = np.zeros((1, N, d), np.float32)
    k = np.zeros((1, N, d), np.float32)
    q[0, :, 0] = sign
    for n in range(N):
        k[0, n, 0] = _tile_of(GRID, TILE, n) + 1
    return q, k


@pytest.mark.parametrize("kh", [1, 5, 11])
def test_topk_keeps_the_largest_scores(kh):
    nT = oracle.num_tiles(GRID, TILE)
    q, k = _ordered_inputs(1.0)
    M = oracle.select_topk(GRID, TILE, q, k, [kh])
    want = np.zeros(nT, np.uint8)
    want[nT - kh:] = 1
    assert all(np.array_equal(M[0, i], want) for i in range(nT))
    q, k = _ordered_inputs(-1.0)
    M = oracle.select_topk(GRID, TILE, q, k, [kh])
    want = np.zeros(nT, np.uint8)
    want[:kh] = 1
    assert all(np.array_equal(M[0, i], want) for i in range(nT))


def test_topk_ties_go_to_the_lower_tile():
    nT = oracle.num_tiles(GRID, TILE)
    N = int(np.prod(GRID))
    rng = np.random.default_rng(5)
    q = np.zeros((2, N, 8), np.float32)  # every score is 0
    k = rng.standard_normal((2, N, 8)).astype(np.float32)
    M = oracle.select_topk(GRID, TILE, q, k, [3, 7])
    for h, kh in enumerate([3, 7]):
        want = np.zeros(nT, np.uint8)
        want[:kh] = 1
        assert all(np.array_equal(M[h, i], want) for i in range(nT))


def test_topk_ends():
    nT = oracle.num_tiles(GRID, TILE)
    N = int(np.prod(GRID))
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, N, 8)).astype(np.float32)
    k = rng.standard_normal((2, N, 8)).astype(np.float32)
    M = oracle.select_topk(GRID, TILE, q, k, [0, nT])
    assert M[0].sum() == 0 and M[1].sum() == nT * nT


def test_topk_matches_the_hunyuan_recipe():
    """The Hunyuan-shaped workload's masks are drawn by this selection (the
    generator's own fp64 numpy code); the oracle must reproduce them."""
    wl = make_workload("hunyuan", heads=3)
    M = oracle.select_topk(wl.grid, wl.tile, wl.q, wl.k, wl.info["k_per_head"])
    assert np.array_equal(M, wl.bitmap.astype(np.uint8))

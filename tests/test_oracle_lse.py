"""Pins of the oracle's log-sum-exp output (AdaSpa page, abstract: the LSE
of each row is the statistic cached across denoising steps): a hand case,
the library logsumexp under an all-ones mask, closed forms when every score
is zero, the additivity of exp(LSE) over disjoint kept sets, an empty row,
and the numpy brute force on ragged grids."""

import json
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import brute
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(x):
    return (bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def _rand(shape, seed, dtype="f32"):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _tile_sizes(grid, tile):
    """Real tokens per tile, by enumerating tokens."""
    T, H, W = grid
    tt, th, tw = tile
    ny, nx = -(-H // th), -(-W // tw)
    sizes = np.zeros(oracle.num_tiles(grid, tile), np.int64)
    for t in range(T):
        for y in range(H):
            for x in range(W):
                sizes[((t // tt) * ny + y // th) * nx + x // tw] += 1
    return sizes


def test_hand_case():
    with open(os.path.join(GOLDEN, "hand_case_lse.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], np.float32)[None]
    k = np.array(g["k"], np.float32)[None]
    v = np.array(g["v"], np.float32)[None]
    O, L = oracle.attention(g["grid"], g["tile"], q, k, v, np.array(g["mask"], np.uint8)[None],
                            scale=g["scale"], threads=1, lse=True)
    assert np.abs(L[0] - np.array(g["expected_lse"])).max() < g["tolerance"]
    O, L = oracle.attention(g["grid"], g["tile"], q, k, v,
                            np.array(g["mask_empty_row1"], np.uint8)[None], scale=g["scale"],
                            threads=1, lse=True)
    assert L[0, 1] == -np.inf and (O[0, 1] == 0).all()
    assert abs(L[0, 0] - g["expected_lse"][0]) < g["tolerance"]


@pytest.mark.parametrize("grid,tile", [((3, 10, 12), (1, 4, 8)), ((2, 5, 7), (2, 2, 3))])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ones_mask_is_library_logsumexp(grid, tile, dtype):
    heads, d = 2, 16
    N = int(np.prod(grid))
    q, k, v = (_rand((heads, N, d), s, dtype) for s in (1, 2, 3))
    nT = oracle.num_tiles(grid, tile)
    _, L = oracle.attention(grid, tile, q, k, v, np.ones((heads, nT, nT), np.uint8), threads=2,
                            lse=True)
    for h in range(heads):
        S = torch.from_numpy(_f64(q)[h]) @ torch.from_numpy(_f64(k)[h]).T / np.sqrt(d)
        assert np.abs(L[h] - logsumexp(S.numpy(), axis=1)).max() < 1e-12


def test_zero_scores_give_log_of_kept_tokens():
    """q = 0: every kept score is 0, so LSE = ln(number of kept real keys)."""
    grid, tile = (3, 10, 12), (1, 4, 8)
    heads, d = 3, 8
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    rng = np.random.default_rng(9)
    M = (rng.random((heads, nT, nT)) < 0.4).astype(np.uint8)
    M[0, 0] = 0  # one empty row
    q = np.zeros((heads, N, d), np.float32)
    k, v = _rand((heads, N, d), 10), _rand((heads, N, d), 11)
    _, L = oracle.attention(grid, tile, q, k, v, M, threads=2, lse=True)
    sizes = _tile_sizes(grid, tile)
    T, H, W = grid
    ny, nx = -(-H // tile[1]), -(-W // tile[2])
    for h in range(heads):
        for n in range(N):
            t, y, x = n // (H * W), (n // W) % H, n % W
            i = ((t // tile[0]) * ny + y // tile[1]) * nx + x // tile[2]
            kept = int((M[h, i].astype(bool) * sizes).sum())
            want = np.log(kept) if kept else -np.inf
            assert L[h, n] == want or abs(L[h, n] - want) < 1e-12, (h, n)


def test_exp_lse_adds_over_disjoint_kept_sets():
    """exp(LSE) is the sum of exp(score) over kept keys, so for disjoint
    kept sets A, B: LSE(A u B) = ln(exp LSE(A) + exp LSE(B))."""
    grid, tile = (2, 8, 12), (1, 4, 4)
    heads, d = 2, 16
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    q, k, v = (_rand((heads, N, d), s, "bf16") for s in (21, 22, 23))
    rng = np.random.default_rng(24)
    side = rng.random((heads, nT, nT)) < 0.5
    A = (side & (rng.random((heads, nT, nT)) < 0.7)).astype(np.uint8)
    B = (~side & (rng.random((heads, nT, nT)) < 0.7)).astype(np.uint8)
    _, LA = oracle.attention(grid, tile, q, k, v, A, threads=2, lse=True)
    _, LB = oracle.attention(grid, tile, q, k, v, B, threads=2, lse=True)
    _, LU = oracle.attention(grid, tile, q, k, v, A | B, threads=2, lse=True)
    want = np.logaddexp(LA, LB)
    fin = np.isfinite(want)
    assert (np.isfinite(LU) == fin).all()
    assert np.abs(LU[fin] - want[fin]).max() < 1e-12


@pytest.mark.parametrize("grid,tile", [((3, 10, 12), (1, 4, 8)), ((5, 3, 3), (2, 3, 3)),
                                       ((1, 1, 5), (1, 1, 8))])
def test_matches_numpy_brute_force(grid, tile):
    heads, d = 3, 8
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    q, k, v = (_rand((heads, N, d), s, "bf16") for s in (31, 32, 33))
    M = (np.random.default_rng(34).random((heads, nT, nT)) < 0.3).astype(np.uint8)
    M[0, 0] = 0
    _, L = oracle.attention(grid, tile, q, k, v, M, threads=2, lse=True)
    ref = brute.lse(grid, tile, _f64(q), _f64(k), M)
    assert (np.isinf(L) == np.isinf(ref)).all()
    fin = np.isfinite(ref)
    assert np.abs(L[fin] - ref[fin]).max() < 1e-12


"""Pins of the oracle's tile mass and dual-window search (Compact Attention
page, Fig. 1 caption: reference attention mass; Fig. 3 and Fig. 4 captions:
windows shrunk from full coverage under recall and cost constraints).

Tile mass: rows sum to one, uniform mass at zero scores, a closed form for
tile-indicator scores, and the recall of a mask equal to the mean over
queries of exp(LSE_mask - LSE_full) from the attention oracle.  Search:
tau = 0 removes everything, tau = 1 keeps everything when every tile pair
carries mass, mass on the own tile leaves exactly the diagonal, axial mass
leaves exactly the cross, and every move left at the end is inadmissible."""

import math

import numpy as np
import pytest

import oracle
from oracle import search

GRID, TILE = (3, 12, 16), (1, 4, 4)  # tile grid 3 x 3 x 4


def _coords():
    a, b, e, shape = search._tile_coords(GRID, TILE)
    return a, b, e, shape


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_tile_mass_rows_sum_to_one_and_uniform_at_zero_scores():
    N = int(np.prod(GRID))
    q, k = _rand((2, N, 8), 1), _rand((2, N, 8), 2)
    A = oracle.tile_mass(GRID, TILE, q, k)
    assert np.abs(A.sum(axis=2) - 1).max() < 1e-12
    counts = oracle.tile_counts(GRID, TILE)
    A0 = oracle.tile_mass(GRID, TILE, np.zeros_like(q), k)
    assert np.abs(A0 - counts[None, None, :] / N).max() < 1e-15


def test_tile_mass_closed_form_for_tile_indicator_scores():
    """q_n = k_n = beta e_tile(n): score beta^2 within a tile, 0 across, so
    A[i, i] = c_i E / (c_i E + N - c_i), A[i, j] = c_j / (c_i E + N - c_i)."""
    grid, tile = (2, 6, 8), (1, 3, 4)  # 2 x 2 x 2 = 8 tiles, some clipped? no: exact
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    _, pos = oracle.perm(grid, tile)
    t_of = pos // int(np.prod(tile))
    beta = 1.5
    x = np.zeros((1, N, nT), np.float32)
    x[0, np.arange(N), t_of] = beta
    A = oracle.tile_mass(grid, tile, x, x, scale=1.0)[0]
    c = oracle.tile_counts(grid, tile).astype(np.float64)
    E = math.exp(beta * beta)
    want = c[None, :] / (c[:, None] * E + N - c[:, None])
    want[np.diag_indices(nT)] = c * E / (c * E + N - c)
    assert np.abs(A - want).max() < 1e-12


def test_recall_equals_mean_retained_mass_from_lse():
    N = int(np.prod(GRID))
    nT = oracle.num_tiles(GRID, TILE)
    q, k, v = _rand((1, N, 8), 3), _rand((1, N, 8), 4), _rand((1, N, 8), 5)
    A = oracle.tile_mass(GRID, TILE, q, k)
    M = (np.random.default_rng(6).random((1, nT, nT)) < 0.4).astype(np.uint8)
    counts = oracle.tile_counts(GRID, TILE)
    recall = float((counts[:, None] * A[0] * M[0]).sum() / counts.sum())
    _, lse_m = oracle.attention(GRID, TILE, q, k, v, M, lse=True)
    _, lse_f = oracle.attention(GRID, TILE, q, k, v, np.ones_like(M), lse=True)
    assert abs(recall - np.exp(lse_m - lse_f).mean()) < 1e-12


GROUPS = [(0, 0), (1, 1), (2, -1)]


def _mask(rows, gph):
    return oracle.mask_from_windows(GRID, TILE, rows, gph)


def test_tau_zero_removes_everything():
    nT = oracle.num_tiles(GRID, TILE)
    A = np.full((1, nT, nT), 1.0 / nT)
    rows, gph, rec, cost = search.search(GRID, TILE, oracle.tile_counts(GRID, TILE), A, [GROUPS], 0.0)
    assert _mask(rows, gph).sum() == 0 and rec[0] == 0 and cost[0] == 0


def test_tau_one_keeps_full_coverage_when_all_pairs_carry_mass():
    nT = oracle.num_tiles(GRID, TILE)
    _, _, _, (nt, ny, nx) = _coords()
    A = np.full((1, nT, nT), 1.0 / nT)
    rows, gph, rec, _ = search.search(GRID, TILE, oracle.tile_counts(GRID, TILE), A, [GROUPS], 1.0)
    assert np.all(rows[:, 2:4] == ny - 1) and np.all(rows[:, 4:6] == nx - 1)
    assert _mask(rows, gph).all() and rec[0] == 1.0


def test_mass_on_the_own_tile_leaves_the_diagonal():
    nT = oracle.num_tiles(GRID, TILE)
    A = np.eye(nT)[None]
    counts = oracle.tile_counts(GRID, TILE)
    rows, gph, rec, cost = search.search(GRID, TILE, counts, A, [GROUPS], 1.0)
    assert np.array_equal(_mask(rows, gph)[0], np.eye(nT, dtype=np.uint8))
    assert rec[0] == 1.0
    assert abs(cost[0] - (counts.astype(float) ** 2).sum() / counts.sum() ** 2) < 1e-15


def test_axial_mass_leaves_the_cross():
    """Mass only on same-frame pairs in the same tile row or column: the
    search must end on exactly that cross (a row band and a column band)."""
    a, b, e, _ = _coords()
    same = (a[:, None] == a[None, :]) & ((b[:, None] == b[None, :]) | (e[:, None] == e[None, :]))
    A = same / same.sum(axis=1, keepdims=True)
    counts = oracle.tile_counts(GRID, TILE)
    rows, gph, rec, _ = search.search(GRID, TILE, counts, A[None], [GROUPS], 1.0)
    assert np.array_equal(_mask(rows, gph)[0], same.astype(np.uint8))
    assert rec[0] == 1.0


@pytest.mark.parametrize("tau,lam", [(0.9, math.inf), (0.95, 4.0), (0.7, 1.5)])
def test_no_admissible_move_is_left(tau, lam):
    N = int(np.prod(GRID))
    q, k = _rand((2, N, 16), 7), _rand((2, N, 16), 8)
    A = oracle.tile_mass(GRID, TILE, q, k)
    counts = oracle.tile_counts(GRID, TILE)
    groups = [GROUPS, [(0, 1), (2, -1)]]
    rows, gph, rec, cost = search.search(GRID, TILE, counts, A, groups, tau, lam)
    off = 0
    _, _, _, (nt, ny, nx) = _coords()
    for h, gh in enumerate(groups):
        assert rec[h] >= tau
        tabs, w_total, c_total = search.tables(GRID, TILE, counts, A[h], gh)
        kept_w = int(round(rec[h] * w_total))
        need = math.ceil(tau * w_total)
        for g in range(len(gh)):
            lo, hi, y, Y, X, x = rows[off + g]
            st = (y, X, Y, x)
            mw, mc = tabs[g]
            cov = search.covered(st, ny, nx)
            for _, new in search.moves(st):
                gone = cov & ~search.covered(new, ny, nx)
                if not gone.any():
                    continue
                dw, dc = int(mw[gone].sum()), int(mc[gone].sum())
                ok = kept_w - dw >= need and (math.isinf(lam) or dw * c_total <= lam * dc * w_total)
                assert not ok, (h, g, st, new)
        off += len(gh)

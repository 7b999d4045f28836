"""Pins for the oracle's slot maps, window-mask evaluation and index lists."""

import numpy as np
import pytest

import oracle
from oracle import brute
from workloads import CONFIGS, accounting, make_workload

GRIDS = [((4, 8, 8), (1, 4, 4)), ((8, 30, 40), (1, 8, 16)), ((3, 10, 12), (1, 4, 8)),
         ((2, 5, 7), (2, 2, 3)), ((1, 1, 5), (1, 1, 8)), ((5, 3, 3), (2, 3, 3)),
         ((21, 45, 80), (1, 8, 16))]


@pytest.mark.parametrize("grid,tile", GRIDS)
def test_perm_matches_enumerated_tile_boxes(oracle_lib, grid, tile):
    perm, pos = oracle.perm(grid, tile)
    B = int(np.prod(tile))
    if int(np.prod(grid)) > 100000:
        pytest.skip("box enumeration only for small grids")
    want = np.full_like(perm, -1)
    for t, box in enumerate(brute.tile_boxes(grid, tile)):
        want[t * B:t * B + len(box)] = box
    assert np.array_equal(perm, want)


@pytest.mark.parametrize("grid,tile", GRIDS)
def test_perm_is_a_bijection_onto_real_slots(oracle_lib, grid, tile):
    perm, pos = oracle.perm(grid, tile)
    N = int(np.prod(grid))
    real = perm >= 0
    assert real.sum() == N
    assert np.array_equal(np.sort(perm[real]), np.arange(N))
    assert np.array_equal(perm[pos], np.arange(N))  # unpermute o permute = id
    # real slots of a tile come first, in increasing token order
    B = int(np.prod(tile))
    counts = oracle.tile_counts(grid, tile)
    blocks = perm.reshape(-1, B)
    for t, c in enumerate(counts):
        assert np.all(blocks[t, :c] >= 0) and np.all(blocks[t, c:] == -1)
        assert np.all(np.diff(blocks[t, :c]) > 0)


def test_pad_slot_counts_of_the_workloads(oracle_lib):
    # nT * B - N for the five workloads: tiny divides evenly; the 720p grids
    # have 45 rows of tokens cut in tiles of 8 (last tile row holds 5).
    want = {"tiny": 0, "small": 2688, "wan": 5040, "hunyuan": 7920, "long": 10080}
    for name, cfg in CONFIGS.items():
        perm, _ = oracle.perm(cfg.grid, cfg.tile)
        assert int((perm < 0).sum()) == want[name], name


def test_tile_counts_sum_and_clipping(oracle_lib):
    c = oracle.tile_counts((21, 45, 80), (1, 8, 16))
    assert c.sum() == 75600 and len(c) == 630
    assert sorted(set(c.tolist())) == [80, 128]
    assert (c == 80).sum() == 105


def test_window_mask_hand_cases(oracle_lib):
    # 2 frames of 3 x 3 tiles (tile 1x1x1).  Group |dt| = 0 has a plus-shaped
    # pair of windows (0, 1) and (1, 0); group |dt| >= 1 keeps only the same
    # position.  Rows worked out by hand.
    grid, tile = (2, 3, 3), (1, 1, 1)
    groups = [[0, 0, 0, 1, 1, 0], [1, -1, 0, -1, 0, -1]]
    M = oracle.mask_from_windows(grid, tile, groups, [2])[0]
    assert sorted(np.nonzero(M[4])[0].tolist()) == [1, 3, 4, 5, 7, 13]  # centre of frame 0
    assert sorted(np.nonzero(M[9])[0].tolist()) == [0, 9, 10, 12]  # corner of frame 1
    # a disabled window (-1) keeps nothing; an unmatched distance keeps nothing
    M2 = oracle.mask_from_windows(grid, tile, [[1, 1, -1, 0, 2, -1]], [1])[0]
    assert M2[4].sum() == 0  # only window 0 could match, it is disabled
    M3 = oracle.mask_from_windows(grid, tile, [[1, 1, 5, -1, 5, -1]], [1])[0]
    assert M3[4].sum() == 9 and all(M3[4, j] for j in range(9, 18))  # other frame only


def _random_specs(rng, heads, tgrid):
    nt, ny, nx = tgrid
    per_head = []
    for _ in range(heads):
        cuts = sorted(rng.choice(np.arange(1, nt + 2), size=2, replace=False))
        bounds = [(0, cuts[0] - 1), (cuts[0], cuts[1] - 1), (cuts[1], -1)]
        groups = []
        for lo, hi in bounds:
            r = rng.integers(-1, max(ny, nx) + 1, size=4)
            groups.append([lo, hi, *r.tolist()])
        per_head.append(groups)
    return per_head


@pytest.mark.parametrize("seed", range(6))
def test_window_mask_counts_match_closed_form(oracle_lib, seed):
    # The number of kept pairs of a dual-window spec has a closed form: along
    # an axis of n tiles a half-extent r < n keeps n (2r + 1) - r (r + 1)
    # pairs, axes multiply, and two windows overlap in the smaller one.
    rng = np.random.default_rng(seed)
    grid, tile = ((5, 30, 40), (1, 8, 16)) if seed % 2 else ((7, 13, 11), (2, 3, 2))
    tgrid = tuple(-(-g // t) for g, t in zip(grid, tile))
    per_head = _random_specs(rng, 4, tgrid)
    groups = [g for ph in per_head for g in ph]
    M = oracle.mask_from_windows(grid, tile, groups, [len(ph) for ph in per_head])
    for h, ph in enumerate(per_head):
        assert int(M[h].sum()) == accounting.window_nnz(ph, tgrid)
        assert np.array_equal(M[h], M[h].T)  # centred windows are symmetric


def test_long_row_window_example(oracle_lib):
    # 42 frames, |dt| <= 4, one row band r = 0 over 6 x 5 tiles: 358 time
    # pairs times 6 * 25 spatial pairs = 53,700 pairs per head.
    M = oracle.mask_from_windows((42, 45, 80), (1, 8, 16), [[0, 4, 0, -1, 4, -1]], [1])
    assert int(M.sum()) == 53700
    assert abs(M.sum() / 1260 ** 2 - 0.03382) < 1e-5


def _check_csr(M, row_ptr, cols, order):
    heads, nT, _ = M.shape
    R = heads * nT
    flat = M.reshape(R, nT)
    lens = np.diff(row_ptr)
    assert row_ptr[0] == 0 and np.array_equal(lens, (flat != 0).sum(axis=1))
    back = np.zeros_like(flat)
    for r in range(R):
        c = cols[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(c) > 0)
        back[r, c] = 1
    assert np.array_equal(back, (flat != 0).astype(np.uint8))
    assert order.tolist() == sorted(range(R), key=lambda r: (-lens[r], r))


@pytest.mark.parametrize("seed", range(4))
def test_csr_round_trips_random_masks(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    M = (rng.random((3, 17, 17)) < [0.0, 0.3, 1.0][seed % 3]).astype(np.uint8) * rng.integers(1, 255)
    _check_csr(M, *oracle.csr(M))


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_csr_of_workload_masks(oracle_lib, name):
    wl = make_workload(name)
    M = oracle.mask_of(wl)
    _check_csr(M, *oracle.csr(M))


@pytest.mark.parametrize("name", ["tiny", "small", "wan", "long"])
def test_oracle_flops_match_accounting(oracle_lib, name):
    wl = make_workload(name, heads=3) if name in ("wan", "long") else make_workload(name)
    M = oracle.mask_of(wl)
    c = oracle.tile_counts(wl.grid, wl.tile)
    assert int(M.sum()) == wl.info["nnz"]
    assert abs(oracle.flops(M, c, wl.head_dim) / wl.info["flops_alg"] - 1.0) < 1e-12

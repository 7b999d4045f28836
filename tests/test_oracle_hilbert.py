"""Pins of the oracle's Hilbert-curve token order (DFSAttn page, abstract:
Hilbert-curve token reordering; construction: the 3D curve of Skilling,
"Programming the Hilbert curve", 2004).

The properties that make a curve a Hilbert curve fix the oracle's: at
order 1 it is the reflected Gray code (t bit first); at every order it is a
bijection onto [0, 8^k) whose consecutive cells are unit steps apart, starts
at the origin, and every aligned run of 8^j indices fills an aligned cube of
side 2^j.  The order of a non-cube grid ranks its cells by that index."""

import numpy as np
import pytest

import oracle


def _cells(k):
    """idx[t, y, x] (index of each cell) and pos[h] (cell of each index)."""
    n = 1 << k
    pos = np.array([oracle.hilbert_point(k, h) for h in range(n ** 3)], dtype=np.int64)
    idx = np.full((n, n, n), -1, dtype=np.int64)
    idx[pos[:, 0], pos[:, 1], pos[:, 2]] = np.arange(n ** 3)
    return idx, pos


def test_order_one_is_the_reflected_gray_code():
    _, pos = _cells(1)
    for i in range(8):
        g = i ^ (i >> 1)
        assert tuple(pos[i]) == ((g >> 2) & 1, (g >> 1) & 1, g & 1)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_bijective_continuous_and_nested(k):
    idx, pos = _cells(k)
    n = 1 << k
    assert pos.min() >= 0 and pos.max() < n
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(n ** 3))
    assert tuple(pos[0]) == (0, 0, 0)
    steps = np.abs(np.diff(pos, axis=0)).sum(axis=1)
    assert np.all(steps == 1)
    for j in range(1, k):
        side, run = 1 << j, 8 ** j
        for m in range(n ** 3 // run):
            block = pos[m * run:(m + 1) * run]
            lo = block.min(axis=0)
            assert np.all(block.max(axis=0) - lo == side - 1)
            assert np.all(lo % side == 0)


@pytest.mark.parametrize("grid", [(3, 5, 7), (1, 6, 10), (4, 4, 4), (2, 9, 3)])
def test_grid_order_ranks_cells_by_cube_index(grid):
    T, H, W = grid
    N = T * H * W
    k = int(np.ceil(np.log2(max(grid)))) if max(grid) > 1 else 0
    seq = oracle.hilbert_order(grid)
    assert np.array_equal(np.sort(seq), np.arange(N))
    idx, _ = _cells(k)
    keys = [idx[n // (H * W), (n // W) % H, n % W] for n in range(N)]
    assert np.array_equal(seq, np.argsort(keys, kind="stable"))


def test_full_cube_grid_order_is_continuous():
    seq = oracle.hilbert_order((8, 8, 8))
    t, y, x = seq // 64, (seq // 8) % 8, seq % 8
    steps = np.abs(np.diff(t)) + np.abs(np.diff(y)) + np.abs(np.diff(x))
    assert np.all(steps == 1)


def test_hilbert_blocks_are_compact():
    """Blocks of 128 consecutive ranks on a 16^3 grid are 4 x 4 x 8 boxes."""
    seq = oracle.hilbert_order((16, 16, 16))
    for b in range(16 ** 3 // 128):
        s = seq[b * 128:(b + 1) * 128]
        ext = sorted(int(v.max() - v.min() + 1) for v in (s // 256, (s // 16) % 16, s % 16))
        assert ext == [4, 4, 8]

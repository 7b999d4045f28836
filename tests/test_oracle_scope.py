"""Pins of the oracle's per-head Top-k estimate (oracle/scope.py; SCOPE
review page, "What carries the argument": the hybrid Top-p / fixed Top-k
base count per query cluster, k_head = ceil(sum n_c b_c / sum n_c), and
r_c = max(b_c, k_head)).  Worked by hand:

- logits ln 4, ln 2, 0, 0 give probabilities 1/2, 1/4, 1/8, 1/8 (all exact
  in binary), so the Top-p counts at rho = 0.5, 0.7, 0.75, 0.76, 0.875, 0.9
  are 1, 2, 2, 3, 3, 4: the threshold is "at least rho", reached exactly
  at 0.75 and 0.875, whatever the order of the logits;
- a weighted average: n = (128, 32), b = (2, 10) gives (256 + 320) / 160 =
  3.6, so k_head = 4 (an unweighted mean would give 6); n = (128, 128,
  64), b = (2, 5, 3) gives 1088 / 320 = 3.4 -> 4; an exact quotient stays:
  n = (128, 128), b = (2, 4) -> 3;
- an end-to-end case on a 1 x 1 x 14 grid cut into tiles of 4 tokens (the
  last one clipped to 2), with every token of a tile equal so that the
  tile means, and the scores, are set by hand.
Each rule is also checked to fail when a plausible mistake is planted."""

import math

import numpy as np
import pytest

import oracle
from oracle import scope

LN = math.log


def test_top_p_counts_worked_by_hand():
    row = np.array([LN(4), LN(2), 0.0, 0.0])
    for rho, want in [(0.5, 1), (0.7, 2), (0.75, 2), (0.76, 3), (0.875, 3), (0.9, 4), (0.0, 0), (1.0, 4)]:
        assert scope.top_p_count(row, rho) == want, rho
        assert scope.top_p_count(row[::-1].copy(), rho) == want, rho
    assert scope.top_p_count(np.zeros(5), 0.6) == 3      # uniform: 0.2 each
    assert scope.top_p_count(np.array([7.0]), 0.3) == 1


def test_head_estimate_worked_by_hand():
    assert scope.head_estimate([2, 10], [128, 32]) == 4
    assert scope.head_estimate([2, 5, 3], [128, 128, 64]) == 4
    assert scope.head_estimate([2, 4], [128, 128]) == 3


def _case():
    """Four query tiles and four key tiles (4, 4, 4, 2 tokens) on a
    1 x 1 x 14 grid, d = 4, scale 1: key tile j is the unit vector e_j and
    query tile i the logits of row i, so s_ij is row i's logit j."""
    grid, tile = (1, 1, 14), (1, 1, 4)
    logits = np.array([[LN(4), LN(2), 0.0, 0.0],      # 1/2 1/4 1/8 1/8
                       [0.0, 0.0, 0.0, 0.0],          # 1/4 each
                       [LN(97), 0.0, 0.0, 0.0],       # 97/100 1/100 ...
                       [0.0, 0.0, LN(2), LN(4)]])     # 1/8 1/8 1/4 1/2
    tile_of = np.arange(14) // 4
    q = logits[tile_of][None].astype(np.float32)
    k = np.eye(4, dtype=np.float32)[tile_of][None]
    return grid, tile, q, k


@pytest.mark.parametrize("rho,k_fixed,base,kh,keep,rows", [
    # rho 0.7: counts 2, 3, 1, 2; k_head = ceil((8 + 12 + 4 + 4) / 14) = 2
    (0.7, 0, [2, 3, 1, 2], 2, [2, 3, 2, 2], [[0, 1], [0, 1, 2], [0, 1], [3, 2]]),
    # rho 0.9: counts 4, 4, 1, 4; k_head = ceil((16 + 16 + 4 + 8) / 14) = ceil(3.14) = 4
    (0.9, 0, [4, 4, 1, 4], 4, [4, 4, 4, 4], [[0, 1, 2, 3]] * 4),
    # fixed floor 2 lifts row 2: counts 2, 3, 2, 2; k_head = ceil(32 / 14) = 3
    (0.7, 2, [2, 3, 2, 2], 3, [3, 3, 3, 3], [[0, 1, 2], [0, 1, 2], [0, 1, 2], [3, 2, 0]]),
])
def test_end_to_end_worked_by_hand(rho, k_fixed, base, kh, keep, rows):
    grid, tile, q, k = _case()
    assert list(oracle.tile_counts(grid, tile)) == [4, 4, 4, 2]
    M, b, khd, kp = scope.select_scope(grid, tile, q, k, rho, k_fixed, scale=1.0)
    assert b[0].tolist() == base and int(khd[0]) == kh and kp[0].tolist() == keep
    for i, js in enumerate(rows):
        want = np.zeros(4, np.uint8)
        want[js] = 1
        assert M[0, i].tolist() == want.tolist(), i


def _planted(monkeypatch, name, fn):
    monkeypatch.setattr(scope, name, fn)


def test_planted_mistakes_fail(monkeypatch):
    row = np.array([LN(4), LN(2), 0.0, 0.0])

    def strict(r, rho):                      # "more than rho" instead of "at least"
        p = np.sort(np.exp(r - r.max()) / np.exp(r - r.max()).sum())[::-1]
        return int(np.searchsorted(np.cumsum(p), rho, side="right") + 1)
    assert strict(row, 0.75) != 2

    def unweighted(base, counts):
        return -(-int(np.sum(base)) // len(base))
    assert unweighted([2, 10], [128, 32]) != 4

    def floor_avg(base, counts):
        return int(np.dot(counts, base)) // int(np.sum(counts))
    assert floor_avg([2, 5, 3], [128, 128, 64]) != 4

    # r_c = min(b_c, k_head) instead of max, or no fixed floor: the
    # end-to-end case's keep counts change.
    grid, tile, q, k = _case()
    s = scope.proxy_scores(grid, tile, q, k, scale=1.0)
    counts = oracle.tile_counts(grid, tile)
    base, kh, keep = scope.scope_counts(s, counts, 0.7, 0)
    assert np.minimum(base, kh[:, None])[0].tolist() != keep[0].tolist()
    base2, _, _ = scope.scope_counts(s, counts, 0.7, 2)
    assert base2[0].tolist() != base[0].tolist()

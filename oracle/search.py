"""The oracle's dual-window mask search (TEST INFRASTRUCTURE ONLY, like the
rest of the oracle).

Compact Attention page, Fig. 3 caption: an offline search shrinks the dual
windows step by step under a recall constraint tau and a cost constraint
lambda and stores the masks; Fig. 4 caption: it starts from full coverage
in every temporal-distance group, and the resulting mask keeps the regions
holding most of each head's attention mass; Fig. 1 caption part (3): two
windows per temporal-distance group.  The pages give no formula; the
reading implemented here:

- Mass: A[h, i, j] from ``oracle.tile_mass`` (full-attention mass of key tile
  j, averaged over the real queries of tile i).  Tile pair (i, j) carries
  weight w = round(A c_i 2^24) (an integer, so sums are exact in any order)
  and cost c_i c_j.  Recall of a head's mask = kept weight / all weight;
  cost = kept cost / N^2.
- Region of a group: offsets (dy, dx) = (|b_i - b_j|, |e_i - e_j|) in tile
  units covered by the union of two origin-anchored rectangles, a wide one
  (y, X) and a tall one (Y, x), -1 <= y <= Y < ny, -1 <= x <= X < nx
  (a rectangle with a negative side covers nothing).  These are the two
  windows of the group: window 0 = (ry y, rx X), window 1 = (ry Y, rx x).
  A pair (i, j) is kept when |a_i - a_j| lies in the group's [dt_lo, dt_hi]
  and its offset is covered.
- Start: every group full, y = Y = ny - 1, x = X = nx - 1.
- Moves of a group, numbered: 0 notch the corner of a rectangle (y = Y and
  x = X: y, x -= 1, removes offset (Y, X)); 1 y -= 1; 2 x -= 1; 3 Y -= 1
  (y = min(y, Y)); 4 X -= 1 (x = min(x, X)).  A move that uncovers no
  offset is not a candidate.
- A candidate is admissible when the recall stays >= tau and its lost
  recall is at most lambda times its saved cost (both as fractions; lambda
  = inf disables this).  Each step applies the admissible candidate of any
  group with the least lost weight per saved cost (a move saving no cost
  loses no weight and ranks first), ties to the larger saved cost, then the
  lower group, then the lower move number; the search ends when none is
  admissible.  Heads are searched independently.
"""

import math

import numpy as np

WEIGHT_SCALE = float(1 << 24)


def _tile_coords(grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    nt, ny, nx = -(-T // tt), -(-H // th), -(-W // tw)
    idx = np.arange(nt * ny * nx)
    return idx // (ny * nx), (idx // nx) % ny, idx % nx, (nt, ny, nx)


def tables(grid, tile, counts, A_h, groups_h):
    """Per group: weight and cost summed by offset (dy, dx), int64 [ny, nx];
    and the head's total weight and cost."""
    a, b, e, (nt, ny, nx) = _tile_coords(grid, tile)
    c = np.asarray(counts, dtype=np.float64)
    w = np.rint(np.asarray(A_h, dtype=np.float64) * c[:, None] * WEIGHT_SCALE).astype(np.int64)
    ci = np.asarray(counts, dtype=np.int64)
    cost = np.outer(ci, ci)
    da = np.abs(a[:, None] - a[None, :])
    dy = np.abs(b[:, None] - b[None, :])
    dx = np.abs(e[:, None] - e[None, :])
    out = []
    for lo, hi in groups_h:
        sel = (da >= lo) & ((hi < 0) | (da <= hi))
        mw = np.zeros((ny, nx), dtype=np.int64)
        mc = np.zeros((ny, nx), dtype=np.int64)
        np.add.at(mw, (dy[sel], dx[sel]), w[sel])
        np.add.at(mc, (dy[sel], dx[sel]), cost[sel])
        out.append((mw, mc))
    return out, int(w.sum()), int(cost.sum())


def covered(state, ny, nx):
    y, X, Y, x = state
    dy = np.arange(ny)[:, None]
    dx = np.arange(nx)[None, :]
    return ((dy <= y) & (dx <= X)) | ((dy <= Y) & (dx <= x))


def moves(state):
    y, X, Y, x = state
    out = []
    if y == Y and x == X and Y >= 0 and X >= 0:
        out.append((0, (y - 1, X, Y, x - 1)))
    if y >= 0:
        out.append((1, (y - 1, X, Y, x)))
    if x >= 0:
        out.append((2, (y, X, Y, x - 1)))
    if Y >= 0:
        out.append((3, (min(y, Y - 1), X, Y - 1, x)))
    if X >= 0:
        out.append((4, (y, X - 1, Y, min(x, X - 1))))
    return out


def _ranks_before(c1, c2):
    """Whether candidate c1 = (dW, dC, g, m) ranks before c2."""
    w1, k1, g1, m1 = c1
    w2, k2, g2, m2 = c2
    if k1 == 0 or k2 == 0:  # a move that saves no cost loses no weight
        if (k1 == 0) != (k2 == 0):
            return k1 == 0
    elif w1 * k2 != w2 * k1:
        return w1 * k2 < w2 * k1
    if k1 != k2:
        return k1 > k2
    return (g1, m1) < (g2, m2)


def _within_cost_bound(dw, dc, w_total, c_total, lam):
    """The cost constraint: the recall a move loses, dw / w_total, is at most
    lam times the cost fraction it saves, dc / c_total (lam = inf: always)."""
    if math.isinf(lam):
        return True
    return float(dw) * float(c_total) <= lam * float(dc) * float(w_total)


def search_head(grid, tile, counts, A_h, groups_h, tau, lam):
    """Returns ([(y, X, Y, x) per group], recall, cost)."""
    _, _, _, (nt, ny, nx) = _tile_coords(grid, tile)
    tabs, w_total, c_total = tables(grid, tile, counts, A_h, groups_h)
    state = [(ny - 1, nx - 1, ny - 1, nx - 1) for _ in groups_h]
    kept_w = sum(int(mw.sum()) for mw, _ in tabs)
    kept_c = sum(int(mc.sum()) for _, mc in tabs)
    need = math.ceil(tau * float(w_total))
    while True:
        best = None
        for g, (mw, mc) in enumerate(tabs):
            cov = covered(state[g], ny, nx)
            for m, new in moves(state[g]):
                gone = cov & ~covered(new, ny, nx)
                if not gone.any():
                    continue
                dw, dc = int(mw[gone].sum()), int(mc[gone].sum())
                if kept_w - dw < need:
                    continue
                if not _within_cost_bound(dw, dc, w_total, c_total, lam):
                    continue
                cand = (dw, dc, g, m)
                if best is None or _ranks_before(cand, best[0]):
                    best = (cand, new)
        if best is None:
            break
        (dw, dc, g, _), new = best
        state[g] = new
        kept_w -= dw
        kept_c -= dc
    return state, kept_w / w_total, kept_c / c_total


def search(grid, tile, counts, A, groups, tau, lam=math.inf):
    """groups: per head a list of (dt_lo, dt_hi).  Returns (spec rows
    [sum of groups, 6] = (dt_lo, dt_hi, ry0, ry1, rx0, rx1) in the window
    group layout, groups_per_head, recall[heads], cost[heads])."""
    rows, gph, rec, cst = [], [], [], []
    for h, gh in enumerate(groups):
        st, r, c = search_head(grid, tile, counts, A[h], gh, tau, lam)
        for (lo, hi), (y, X, Y, x) in zip(gh, st):
            rows.append((lo, hi, y, Y, X, x))
        gph.append(len(gh))
        rec.append(r)
        cst.append(c)
    return (np.array(rows, dtype=np.int32).reshape(-1, 6), np.array(gph, dtype=np.int32),
            np.array(rec), np.array(cst))

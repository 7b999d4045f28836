"""The oracle's online per-head Top-k estimate for tile selection (TEST
INFRASTRUCTURE ONLY, like the rest of the oracle).

SCOPE review page ("What carries the argument", and the summary): a hybrid
Top-p / fixed-Top-k selection gives each query cluster c a base count b_c
of retained keys; the head's estimate is the query-size-weighted average
k_head = ceil(sum_c n_c b_c / sum_c n_c) (its Eq. 9), and only the clusters
whose base count falls below it are extended: r_c = max(b_c, k_head) (its
Eq. 10).  The page's fixed Top-k floor is a ratio alpha = 0.1 of the keys;
here it is an input count k_fixed (key tiles; ceil(0.1 nT) for the page's
ratio), and the Top-p threshold rho, which the page does not report, is an
input too.  The reading at the granularity of this library (the pages apply
it per key; here, as in the block-level proxy of the tile selection, per
tile):

- a query cluster is a query tile, n_c its real tokens;
- the proxy logits of row c are s_cj = scale * qbar_c . kbar_j over all key
  tiles j (qbar, kbar: means of the tiles' real tokens), and the Top-p
  distribution is their softmax over j, one entry per key tile;
- Top-p count p_c = the smallest m such that the m largest probabilities
  sum to at least rho (0 when rho <= 0, every tile when rho >= 1);
- base count b_c = min(nT, max(p_c, k_fixed));
- row c then keeps its r_c highest-scoring key tiles, ties to the lower j
  (the same order as the per-head top-k selection).

Everything is fp64; the counts and the weighted average are exact integer
arithmetic.
"""

import math

import numpy as np

from . import num_tiles, tile_counts, tile_means


def proxy_scores(grid, tile, q, k, scale=None):
    """s[h, i, j] = scale * qbar_i . kbar_j, fp64."""
    heads, _, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = []
    for h in range(heads):
        qb = tile_means(grid, tile, q[h])
        kb = tile_means(grid, tile, k[h])
        out.append(scale * (qb @ kb.T))
    return np.stack(out)


def top_p_count(row, rho):
    """The smallest m such that the m largest softmax probabilities of the
    logits in `row` sum to at least rho."""
    n = row.shape[0]
    if rho <= 0.0:
        return 0
    if rho >= 1.0:
        return n
    p = np.exp(row - row.max())
    p = np.sort(p / p.sum())[::-1]
    cum = np.cumsum(p)
    return int(min(n, np.searchsorted(cum, rho, side="left") + 1))


def head_estimate(base, counts):
    """k_head = ceil(sum_c n_c b_c / sum_c n_c), exact."""
    num = int(np.dot(np.asarray(counts, dtype=np.int64), np.asarray(base, dtype=np.int64)))
    den = int(np.sum(np.asarray(counts, dtype=np.int64)))
    return -(-num // den)


def scope_counts(scores, counts, rho, k_fixed):
    """(base [heads, nT], k_head [heads], keep [heads, nT]) from the proxy
    scores and the query tiles' real token counts."""
    heads, nT, _ = scores.shape
    base = np.empty((heads, nT), dtype=np.int64)
    for h in range(heads):
        for i in range(nT):
            base[h, i] = min(nT, max(top_p_count(scores[h, i], rho), k_fixed))
    kh = np.array([head_estimate(base[h], counts) for h in range(heads)], dtype=np.int64)
    keep = np.maximum(base, kh[:, None])
    return base, kh, keep


def select_rows(scores, keep):
    """Bitmap [heads, nT, nT]: row i of head h keeps its keep[h, i]
    highest-scoring key tiles, ties to the lower j."""
    heads, nT, _ = scores.shape
    M = np.zeros((heads, nT, nT), dtype=np.uint8)
    j = np.arange(nT)
    for h in range(heads):
        for i in range(nT):
            order = np.lexsort((j, -scores[h, i]))
            M[h, i, order[:keep[h, i]]] = 1
    return M


def select_scope(grid, tile, q, k, rho, k_fixed, scale=None):
    """The whole selection: (bitmap, base, k_head, keep)."""
    s = proxy_scores(grid, tile, q, k, scale)
    base, kh, keep = scope_counts(s, tile_counts(grid, tile), rho, k_fixed)
    assert s.shape[1] == num_tiles(grid, tile)
    return select_rows(s, keep), base, kh, keep

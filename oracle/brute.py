"""numpy fp64 brute force for small grids (test infrastructure).

An independent second rendering of the oracle's definition: it enumerates
each tile's token box by coordinate ranges, expands the tile mask into the
full N x N token mask, and evaluates masked softmax attention with whole
matrices.  Used to cross-check the C oracle on small grids.
"""

import numpy as np


def tile_boxes(grid, tile):
    """Token ids of each tile, tiles raster over (t, y, x), each box in
    raster token order."""
    T, H, W = grid
    tt, th, tw = tile
    boxes = []
    for a in range(0, T, tt):
        for b in range(0, H, th):
            for e in range(0, W, tw):
                ids = [(t * H + y) * W + x
                       for t in range(a, min(a + tt, T))
                       for y in range(b, min(b + th, H))
                       for x in range(e, min(e + tw, W))]
                boxes.append(np.array(ids, dtype=np.int64))
    return boxes


def token_mask(grid, tile, Mh):
    """Expand one head's tile mask [nT, nT] into a boolean [N, N] token mask."""
    boxes = tile_boxes(grid, tile)
    N = int(np.prod(grid))
    out = np.zeros((N, N), dtype=bool)
    for i, bi in enumerate(boxes):
        for j, bj in enumerate(boxes):
            if Mh[i, j]:
                out[np.ix_(bi, bj)] = True
    return out


def attention(grid, tile, q, k, v, M, scale=None):
    """q, k, v: float64 [heads, N, d]; M: [heads, nT, nT]. Returns [heads, N, d]."""
    heads, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((heads, N, d))
    for h in range(heads):
        keep = token_mask(grid, tile, M[h])
        S = scale * (q[h] @ k[h].T)
        S = np.where(keep, S, -np.inf)
        rows = keep.any(axis=1)
        mu = np.where(rows, S.max(axis=1), 0.0)
        E = np.where(keep, np.exp(S - mu[:, None]), 0.0)
        den = E.sum(axis=1)
        P = np.divide(E, den[:, None], out=np.zeros_like(E), where=den[:, None] > 0)
        out[h] = P @ v[h]
    return out


def lse(grid, tile, q, k, M, scale=None):
    """Log-sum-exp of each query's kept scores: [heads, N], -inf where a row
    keeps nothing."""
    heads, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((heads, N), -np.inf)
    for h in range(heads):
        keep = token_mask(grid, tile, M[h])
        S = scale * (q[h] @ k[h].T)
        for n in range(N):
            if keep[n].any():
                s = S[n, keep[n]]
                out[h, n] = s.max() + np.log(np.exp(s - s.max()).sum())
    return out

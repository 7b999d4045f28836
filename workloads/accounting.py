"""Counting for the synthetic workloads: kept tile pairs, densities and
algorithmic FLOPs.

These are bookkeeping formulas used to steer mask recipes to their density
targets and to report throughput.  They never decide which tile pairs a
kernel or the oracle keeps.

Dual-window specs are separable: a pair (i, j) is kept when the tile-t
distance |a_i - a_j| lies in one of the head's groups and (|b_i - b_j|,
|e_i - e_j|) lies in the union of that group's two windows.  So every count
is a sum over groups of (time-pair sum) x (spatial-union sum), and the union
of two centred windows is |W0| + |W1| - |W0 and W1|, where the intersection is
the window with the smaller half-extent on each axis.

FLOP convention: scores and the weighted sum each cost 2 d per (query, key)
pair, so one kept pair of tiles with c_i and c_j real tokens costs
4 d c_i c_j.  Dense attention over N tokens costs 4 N^2 d per head, the
convention behind the AdaSpa page's budget of about 500 PFLOP of attention
for an 8-second 720p HunyuanVideo clip (abstract).
"""

import numpy as np


def _axis_counts(n_tokens, t):
    n = -(-n_tokens // t)
    return np.minimum(t, n_tokens - t * np.arange(n)).astype(np.float64)


def tile_counts(grid, tile):
    """Real tokens per tile, tile ids raster over (t, y, x): [nT] int64."""
    ct, cy, cx = (_axis_counts(g, t) for g, t in zip(grid, tile))
    return np.einsum("a,b,e->abe", ct, cy, cx).reshape(-1).astype(np.int64)


def _dist(n):
    i = np.arange(n)
    return np.abs(i[:, None] - i[None, :])


def _band_sum(w, r):
    """sum over index pairs with |i - j| <= r of w_i w_j (r < 0: empty)."""
    if r < 0:
        return 0.0
    D = _dist(len(w))
    return float(w @ ((D <= r) * 1.0) @ w)


def _time_sum(w, lo, hi):
    D = _dist(len(w))
    sel = D >= lo
    if hi >= 0:
        sel &= D <= hi
    return float(w @ (sel * 1.0) @ w)


def _union_sum(wy, wx, ry0, ry1, rx0, rx1):
    on0 = ry0 >= 0 and rx0 >= 0
    on1 = ry1 >= 0 and rx1 >= 0
    s = 0.0
    if on0:
        s += _band_sum(wy, ry0) * _band_sum(wx, rx0)
    if on1:
        s += _band_sum(wy, ry1) * _band_sum(wx, rx1)
    if on0 and on1:
        s -= _band_sum(wy, min(ry0, ry1)) * _band_sum(wx, min(rx0, rx1))
    return s


def window_pair_sum(groups, wt, wy, wx):
    """sum over kept tile pairs of one head of w(i) w(j), w separable."""
    total = 0.0
    for lo, hi, ry0, ry1, rx0, rx1 in groups:
        total += _time_sum(wt, lo, hi) * _union_sum(wy, wx, ry0, ry1, rx0, rx1)
    return total


def window_nnz(groups, tgrid):
    nt, ny, nx = tgrid
    return int(round(window_pair_sum(groups, np.ones(nt), np.ones(ny), np.ones(nx))))


def window_nnz_total(per_head, tgrid):
    return sum(window_nnz(g, tgrid) for g in per_head)


def _per_head_groups(wl):
    out, off = [], 0
    for n in wl.groups_per_head:
        out.append([tuple(int(x) for x in row) for row in wl.groups[off:off + n]])
        off += n
    return out


def summarize(wl):
    """Kept tile pairs, densities and FLOPs of a workload's mask."""
    grid, tile, d = wl.config.grid, wl.config.tile, wl.config.head_dim
    tgrid = tuple(-(-g // t) for g, t in zip(grid, tile))
    nT = int(np.prod(tgrid))
    B = int(np.prod(tile))
    N = int(np.prod(grid))
    ct, cy, cx = (_axis_counts(g, t) for g, t in zip(grid, tile))
    if wl.mask_kind == "bitmap":
        c = tile_counts(grid, tile).astype(np.float64)
        nnz_h = [int(np.count_nonzero(wl.bitmap[h])) for h in range(wl.heads)]
        pair_h = [float(c @ (wl.bitmap[h] != 0).astype(np.float64) @ c) for h in range(wl.heads)]
    else:
        per_head = _per_head_groups(wl)
        nnz_h = [window_nnz(g, tgrid) for g in per_head]
        pair_h = [window_pair_sum(g, ct, cy, cx) for g in per_head]
    nnz = int(sum(nnz_h))
    pairs = float(sum(pair_h))
    return {
        "nT": nT,
        "tile_volume": B,
        "tokens": N,
        "nnz": nnz,
        "nnz_per_head": nnz_h,
        "tile_density": nnz / (wl.heads * nT * nT),
        "token_density": pairs / (wl.heads * float(N) * N),
        "flops_alg": 4.0 * d * pairs,
        "flops_issued": 4.0 * d * B * B * nnz,
        "flops_dense": 4.0 * d * float(N) * N * wl.heads,
    }

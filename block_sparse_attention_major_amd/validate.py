"""Host-side validation of a compiled mask (a debugging aid).

``check_compiled_mask(h)`` reads the index lists the GPU mask compiler wrote
(through the sparse_attn_read_index_lists / read_pair_lists hooks) and checks
their structure on the host, without any reference implementation:

  row lists  (one per query tile, r = h nT + i)
    - row_ptr starts at 0, never decreases, and ends at the kept-pair count
      (a mask that overflowed its list capacity is itself reported);
    - every row's key tiles are in [0, nT) and strictly ascending;
    - the work order is a permutation of the rows sorted by decreasing
      length, ties by row id;
  pair lists (matrix-core kernel only; one per pair of neighbouring query
  tiles along the layout's pair axis)
    - a pair the pair kernel serves (flag 1) lists the ascending union of its
      two tiles' rows, each entry carrying the key tile, its real token count
      and which of the two tiles keeps it; a pair it does not serve (flag 0)
      is empty;
    - the flag follows the layout's pairing: under OVERLAP a pair is served
      when the union is at most 7/10 of the two rows' total length (an empty
      pair is served), under ALL always, under NONE never;
    - the pair work order is sorted like the row order.

It raises ValueError naming the first violation and returns a small summary
otherwise.  The lists live on the device; this copies them to the host, so
use it in tests and debugging, not in a timed loop.
"""

import numpy as np

from . import (SPARSE_ATTN_KERNEL_MFMA_BF16, SPARSE_ATTN_ORDER_HILBERT, SPARSE_ATTN_PAIRING_ALL,
               SPARSE_ATTN_PAIRING_NONE, sparse_attn_layout,
               sparse_attn_mask_info, sparse_attn_read_index_lists, sparse_attn_read_pair_lists)

PAIR_NUM, PAIR_DEN = 7, 10


def _tile_counts(h, L):
    """Real tokens per tile from the handle's grid and tile shape."""
    nT, B = L["tiles"], L["tile_volume"]
    if L["order"] == SPARSE_ATTN_ORDER_HILBERT:
        c = np.full(nT, B, np.int64)
        c[-1] = L["tokens"] - (nT - 1) * B
        return c
    T, H, W = h.cfg.grid
    tt, th, tw = h.cfg.tile
    nt, ny, nx = L["tile_grid"]
    a = np.arange(nT) // (ny * nx)
    b = (np.arange(nT) // nx) % ny
    e = np.arange(nT) % nx
    return (np.minimum(tt, T - a * tt) * np.minimum(th, H - b * th) * np.minimum(tw, W - e * tw)).astype(np.int64)


def _pair_tiles(L, pr):
    """Query tiles (t1, t2) of pair pr of one head (t2 = -1: alone)."""
    nt, ny, nx = L["tile_grid"]
    pn = L["pair_grid"]
    ax = L["pair_axis"]
    a, b, e = pr // (pn[1] * pn[2]), (pr // pn[2]) % pn[1], pr % pn[2]
    c1 = [a, b, e]
    c2 = [a, b, e]
    two = False
    if ax >= 0:
        c1[ax] = 2 * c1[ax]
        c2[ax] = c1[ax] + 1
        two = c2[ax] < (nt, ny, nx)[ax]
    t1 = (c1[0] * ny + c1[1]) * nx + c1[2]
    t2 = (c2[0] * ny + c2[1]) * nx + c2[2] if two else -1
    return t1, t2


def _check_order(order, lengths, what):
    R = lengths.shape[0]
    if sorted(order.tolist()) != list(range(R)):
        raise ValueError(f"{what}: the work order is not a permutation of the {R} rows")
    key = np.lexsort((np.arange(R), -lengths))
    if not np.array_equal(order, key):
        bad = int(np.nonzero(order != key)[0][0])
        raise ValueError(f"{what}: work order position {bad} holds row {int(order[bad])}, expected {int(key[bad])}")


def check_row_lists(rp, cl, od, nT, nnz):
    """Row lists (row_ptr [R + 1], cols [nnz], order [R]) of R = len(od)
    query tiles over nT key tiles; returns the per-row key-tile arrays."""
    rp, cl, od = (np.asarray(x, dtype=np.int64) for x in (rp, cl, od))
    R = od.shape[0]
    if rp.shape[0] != R + 1 or rp[0] != 0 or np.any(np.diff(rp) < 0):
        raise ValueError("row_ptr does not start at 0, has the wrong length or decreases")
    if rp[R] != nnz or cl.shape[0] < nnz:
        raise ValueError(f"row_ptr ends at {rp[R]}, the mask keeps {nnz} pairs")
    rows = []
    for r in range(R):
        seg = cl[rp[r]:rp[r + 1]]
        if seg.size and (seg.min() < 0 or seg.max() >= nT):
            raise ValueError(f"row {r}: key tile outside [0, {nT})")
        if np.any(np.diff(seg) <= 0):
            raise ValueError(f"row {r}: key tiles not strictly ascending")
        rows.append(seg)
    _check_order(od, np.diff(rp), "rows")
    return rows


def check_pair_lists(rows, prp, pcl, pod, pfl, L, counts, heads):
    """Pair lists against the row lists they merge; returns the number of
    pairs the pair kernel serves."""
    prp, pcl, pod, pfl = (np.asarray(x, dtype=np.int64) for x in (prp, pcl, pod, pfl))
    nT, npairs = L["tiles"], L["pairs"]
    P = heads * npairs
    if prp.shape[0] != P + 1 or prp[0] != 0 or np.any(np.diff(prp) < 0):
        raise ValueError("pair row_ptr does not start at 0, has the wrong length or decreases")
    served = 0
    for p in range(P):
        hh, pr = divmod(p, npairs)
        t1, t2 = _pair_tiles(L, pr)
        r1 = rows[hh * nT + t1]
        r2 = rows[hh * nT + t2] if t2 >= 0 else np.zeros(0, np.int64)
        union = np.union1d(r1, r2)
        if L["pairing"] == SPARSE_ATTN_PAIRING_ALL:
            accept = True
        elif L["pairing"] == SPARSE_ATTN_PAIRING_NONE:
            accept = False
        else:
            accept = union.size * PAIR_DEN <= PAIR_NUM * (r1.size + r2.size)
        if pfl[p] != int(accept):
            raise ValueError(f"pair {p}: flag {pfl[p]}, the sharing rule gives {int(accept)}")
        seg = pcl[prp[p]:prp[p + 1]]
        if not accept:
            if seg.size:
                raise ValueError(f"pair {p}: not served by the pair kernel but its list is not empty")
            continue
        served += 1
        bits = np.isin(union, r1).astype(np.int64) | (np.isin(union, r2).astype(np.int64) << 1)
        want = union | (counts[union] << 16) | (bits << 24)
        if not np.array_equal(seg, want):
            raise ValueError(f"pair {p} (tiles {t1}, {t2}): entries differ from the union of its rows")
    _check_order(pod, np.diff(prp), "pairs")
    return served


def check_compiled_mask(h, stream=None):
    """Reads the handle's compiled lists back and checks them (see the
    module docstring); returns a summary dict or raises ValueError."""
    import torch

    L = sparse_attn_layout(h)
    heads, nT = h.cfg.heads, L["tiles"]
    R = heads * nT
    nnz, overflow = sparse_attn_mask_info(h, stream)
    if overflow:
        raise ValueError(f"the index list overflowed its capacity ({nnz} kept pairs)")
    i32 = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device="cuda")
    row_ptr, cols, order = i32(R + 1), i32(nnz), i32(R)
    sparse_attn_read_index_lists(h, row_ptr, cols, order, stream)
    torch.cuda.synchronize()
    host = lambda t, n: t.cpu().numpy().astype(np.int64)[:n]
    rows = check_row_lists(host(row_ptr, R + 1), host(cols, nnz), host(order, R), nT, int(nnz))
    summary = {"rows": R, "nnz": int(nnz)}
    if L["kernel"] != SPARSE_ATTN_KERNEL_MFMA_BF16:
        return summary
    P = heads * L["pairs"]
    prp, pcl, pod, pfl = i32(P + 1), i32(nnz), i32(P), i32(P)
    sparse_attn_read_pair_lists(h, prp, pcl, pod, pfl, stream)
    torch.cuda.synchronize()
    pn = int(host(prp, P + 1)[P])
    served = check_pair_lists(rows, host(prp, P + 1), host(pcl, pn), host(pod, P), host(pfl, P), L,
                              _tile_counts(h, L), heads)
    summary.update({"pairs": P, "pairs_served": served})
    return summary

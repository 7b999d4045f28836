"""fp64 CPU oracle for tile-masked video attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It
shares no code with the GPU library.  ``oracle.c`` states the definitions and
the passages of the pages they follow; ``brute`` is an independent numpy
rendering used to cross-check it on small grids.
"""

import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None


class _Grid(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("T", "H", "W", "tt", "th", "tw")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        lib = ctypes.CDLL(LIB)
        P = ctypes.POINTER
        g = P(_Grid)
        lib.oracle_num_tiles.argtypes = [g]
        lib.oracle_num_tiles.restype = ctypes.c_int64
        lib.oracle_tile_counts.argtypes = [g, ctypes.c_void_p]
        lib.oracle_perm.argtypes = [g, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_mask_from_windows.argtypes = [g, ctypes.c_int64, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_csr.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_csr.restype = ctypes.c_int64
        lib.oracle_attention_rows.argtypes = [g, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int]
        lib.oracle_probabilities.argtypes = [g, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                             ctypes.c_void_p]
        lib.oracle_tile_means.argtypes = [g, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
        lib.oracle_select_topk.argtypes = [g, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_hilbert_point.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.POINTER(ctypes.c_int64),
                                             ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        lib.oracle_hilbert_point.restype = None
        lib.oracle_hilbert_order.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p]
        lib.oracle_tile_mass.argtypes = [g, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int]
        _lib = lib
    return _lib


def _grid(grid, tile):
    return _Grid(*(int(x) for x in grid), *(int(x) for x in tile))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x):
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.uint16:
        return 1
    raise TypeError("inputs must be float32 or uint16 (bfloat16 bits)")


def num_tiles(grid, tile):
    return int(_load().oracle_num_tiles(ctypes.byref(_grid(grid, tile))))


def tile_counts(grid, tile):
    out = np.empty(num_tiles(grid, tile), dtype=np.int64)
    _load().oracle_tile_counts(ctypes.byref(_grid(grid, tile)), _ptr(out))
    return out


def perm(grid, tile):
    """(perm[nT * B], pos[N]): token of each tile-major slot (-1 = empty)
    and slot of each token."""
    nT = num_tiles(grid, tile)
    B = int(np.prod(tile))
    N = int(np.prod(grid))
    p = np.empty(nT * B, dtype=np.int64)
    q = np.empty(N, dtype=np.int64)
    _load().oracle_perm(ctypes.byref(_grid(grid, tile)), _ptr(p), _ptr(q))
    return p, q


def hilbert_point(k, h):
    """Cell (t, y, x) at index h of the 3D Hilbert curve over a 2^k cube."""
    t, y, x = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _load().oracle_hilbert_point(int(k), int(h), ctypes.byref(t), ctypes.byref(y), ctypes.byref(x))
    return t.value, y.value, x.value


def hilbert_order(grid):
    """seq[N]: raster token of each Hilbert rank (cube points outside the
    grid skipped).  Runs of B consecutive ranks are the blocks of the
    Hilbert layout, i.e. the tiles of a (1, 1, N) grid with tile (1, 1, B)
    over the tokens taken in this order."""
    T, H, W = (int(v) for v in grid)
    seq = np.empty(T * H * W, dtype=np.int64)
    _load().oracle_hilbert_order(T, H, W, _ptr(seq))
    return seq


def mask_from_windows(grid, tile, groups, groups_per_head):
    groups = np.ascontiguousarray(groups, dtype=np.int32).reshape(-1, 6)
    gph = np.ascontiguousarray(groups_per_head, dtype=np.int32)
    nT = num_tiles(grid, tile)
    M = np.empty((len(gph), nT, nT), dtype=np.uint8)
    _load().oracle_mask_from_windows(ctypes.byref(_grid(grid, tile)), len(gph), _ptr(groups),
                                     _ptr(gph), _ptr(M))
    return M


def mask_of(wl):
    """Dense tile mask of a workload, evaluated by the oracle."""
    if wl.mask_kind == "bitmap":
        return np.ascontiguousarray(wl.bitmap != 0, dtype=np.uint8)
    return mask_from_windows(wl.grid, wl.tile, wl.groups, wl.groups_per_head)


def csr(M):
    """(row_ptr, cols, order) of a dense tile mask [heads, nT, nT]."""
    M = np.ascontiguousarray(M, dtype=np.uint8)
    heads, nT, _ = M.shape
    R = heads * nT
    row_ptr = np.empty(R + 1, dtype=np.int64)
    lib = _load()
    nnz = lib.oracle_csr(_ptr(M), heads, nT, _ptr(row_ptr), None, None)
    cols = np.empty(max(nnz, 1), dtype=np.int64)
    order = np.empty(max(R, 1), dtype=np.int64)
    lib.oracle_csr(_ptr(M), heads, nT, _ptr(row_ptr), _ptr(cols), _ptr(order))
    return row_ptr, cols[:nnz], order[:R]


def default_threads():
    return len(os.sched_getaffinity(0))


def attention_rows(grid, tile, q, k, v, M, rows, scale=None, threads=None, lse=False):
    """fp64 outputs of the given flattened query rows (h * N + n): [len(rows), d].
    With lse=True also the rows' log-sum-exp of kept scores (natural log,
    -inf for a row that keeps nothing): returns (out, lse)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k, v must share a dtype")
    heads, N, d = q.shape
    M = np.ascontiguousarray(M, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((len(rows), d), dtype=np.float64)
    L = np.empty(len(rows), dtype=np.float64) if lse else None
    _load().oracle_attention_rows(ctypes.byref(_grid(grid, tile)), heads, d, code, _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(M), float(scale), _ptr(rows), len(rows), _ptr(out),
                                  _ptr(L) if lse else None, int(threads or default_threads()))
    return (out, L) if lse else out


def attention(grid, tile, q, k, v, M, scale=None, threads=None, lse=False):
    """fp64 outputs of every query: [heads, N, d] (with lse=True also the
    log-sum-exp [heads, N])."""
    heads, N, d = q.shape
    rows = np.arange(heads * N, dtype=np.int64)
    r = attention_rows(grid, tile, q, k, v, M, rows, scale, threads, lse)
    if lse:
        return r[0].reshape(heads, N, d), r[1].reshape(heads, N)
    return r.reshape(heads, N, d)


def probabilities(grid, tile, q, k, Mh, scale=None):
    """Attention weights of one head on a small grid: [N, N] fp64."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    P = np.empty((N, N), dtype=np.float64)
    _load().oracle_probabilities(ctypes.byref(_grid(grid, tile)), d, _dtype_code(q), _ptr(q), _ptr(k),
                                 _ptr(np.ascontiguousarray(Mh, dtype=np.uint8)), float(scale), _ptr(P))
    return P


def tile_means(grid, tile, x):
    """fp64 mean of each tile's real tokens: x [N, d] -> [nT, d]."""
    x = np.ascontiguousarray(x)
    N, d = x.shape
    out = np.empty((num_tiles(grid, tile), d), dtype=np.float64)
    _load().oracle_tile_means(ctypes.byref(_grid(grid, tile)), d, _dtype_code(x), _ptr(x), _ptr(out))
    return out


def select_topk(grid, tile, q, k, kh, scale=None, threads=None):
    """Tile mask [heads, nT, nT]: row i of head h keeps the kh[h] key tiles
    with the largest mean-pooled score scale * qbar_i . kbar_j, ties to the
    lower j."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    heads, N, d = q.shape
    if _dtype_code(k) != _dtype_code(q):
        raise TypeError("q, k must share a dtype")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nT = num_tiles(grid, tile)
    kh = np.ascontiguousarray(kh, dtype=np.int64)
    M = np.empty((heads, nT, nT), dtype=np.uint8)
    _load().oracle_select_topk(ctypes.byref(_grid(grid, tile)), heads, d, _dtype_code(q), _ptr(q),
                               _ptr(k), _ptr(kh), float(scale), _ptr(M),
                               int(threads or default_threads()))
    return M


def flops(M, counts, d):
    """Algorithmic FLOPs 4 d sum over kept tile pairs of c_i c_j."""
    c = np.asarray(counts, dtype=np.float64)
    return 4.0 * d * sum(float(c @ (M[h] != 0).astype(np.float64) @ c) for h in range(M.shape[0]))


def tile_mass(grid, tile, q, k, qtiles=None, scale=None, threads=None):
    """Full-attention mass per tile pair, fp64: A[h, i, j] = mean over the
    real queries of tile i of the softmax mass (over all keys) on tile j.
    qtiles: flattened h * nT + i to evaluate (default all) -> [len, nT];
    with qtiles None the result is [heads, nT, nT]."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    heads, N, d = q.shape
    if _dtype_code(k) != _dtype_code(q):
        raise TypeError("q, k must share a dtype")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nT = num_tiles(grid, tile)
    full = qtiles is None
    qt = np.arange(heads * nT, dtype=np.int64) if full else np.ascontiguousarray(qtiles, dtype=np.int64)
    out = np.empty((len(qt), nT), dtype=np.float64)
    _load().oracle_tile_mass(ctypes.byref(_grid(grid, tile)), heads, d, _dtype_code(q), _ptr(q),
                             _ptr(k), float(scale), _ptr(qt), len(qt), _ptr(out),
                             int(threads or default_threads()))
    return out.reshape(heads, nT, nT) if full else out

"""GPU tile selection with the per-head Top-k estimate
(sparse_attn_select_scope) against the oracle (oracle/scope.py; SCOPE
review page, "What carries the argument": hybrid Top-p / fixed Top-k base
counts, k_head = ceil(sum n_c b_c / sum n_c), r_c = max(b_c, k_head)).

The GPU takes the Top-p decision in fp32, the oracle in fp64, so a row
whose cumulative mass crosses rho within fp32 rounding may get a count one
off.  Every GPU base count must be one the oracle's sorted probabilities
allow within a tolerance derived from the arithmetic (see _mass_tol), and
such rows stay rare (at most 1 per 100).  Given the GPU's base counts,
k_head and the final counts are exact integer arithmetic and are checked
exactly; each row then keeps exactly its count, and any tile chosen
differently from the oracle's top-r order must be a score near-tie within
score_error_bound (as for the plain top-k selection)."""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from oracle import scope
from workloads import make_workload

from gpu_helpers import dev
from test_gpu_select import score_error_bound

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _gpu(h, q, k, rho, k_fixed):
    L = sa.sparse_attn_layout(h)
    heads, nT = q.shape[0], L["tiles"]
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    qd, kd = dev(q), dev(k)
    sa.sparse_attn_permute_inputs(h, qd, kd, kd, ws)
    bm = torch.full((heads, nT, nT), 7, dtype=torch.uint8, device="cuda")
    base = torch.full((heads, nT), -5, dtype=torch.int32, device="cuda")
    keep = torch.full((heads, nT), -5, dtype=torch.int32, device="cuda")
    sa.sparse_attn_select_scope(h, rho, k_fixed, ws, bm, base=base, keep=keep)
    torch.cuda.synchronize()
    return bm.cpu().numpy(), base.cpu().numpy().astype(np.int64), keep.cpu().numpy().astype(np.int64)


def _mass_tol(E_row, span, nT):
    """Bound on the error of a cumulative softmax mass computed in fp32 from
    scores with absolute errors <= E: each probability e^(s_j - max) / Z
    moves by at most a relative 2 E (its own score and, through Z, the
    others'), 2 span u from rounding the exponent (s_j - max) log2 e (span:
    the row's score range) and the exponential's few ulp; the fp32 sums of
    up to nT positive terms add nT u relative.  Masses are at most 1, so
    this is an absolute bound; doubled for the second-order terms."""
    return 2.0 * (2.0 * E_row + 2.0 * span * U + 4 * U + nT * U)


def _allowed_counts(row_scores, rho, tol):
    """The Top-p counts m whose cumulative mass the fp64 probabilities put
    within tol of the rho crossing."""
    n = row_scores.shape[0]
    if rho <= 0:
        return {0}
    if rho >= 1:
        return {n}
    p = np.exp(row_scores - row_scores.max())
    cum = np.concatenate([[0.0], np.cumsum(np.sort(p / p.sum())[::-1])])
    return {m for m in range(1, n + 1) if cum[m] >= rho - tol and cum[m - 1] < rho + tol}


def _check(grid, tile, q, k, rho, k_fixed):
    heads, _, d = q.shape
    h = sa.sparse_attn_create(heads, d, grid, tile, "f32" if q.dtype == np.float32 else "bf16")
    M, base, keep = _gpu(h, q, k, rho, k_fixed)
    S = scope.proxy_scores(grid, tile, q, k)
    nT = S.shape[1]
    counts = oracle.tile_counts(grid, tile)
    want_base, want_kh, want_keep = scope.scope_counts(S, counts, rho, k_fixed)
    E = score_error_bound(grid, tile, q, k, d)
    off = 0
    for hh in range(heads):
        for i in range(nT):
            if base[hh, i] != want_base[hh, i]:
                off += 1
                tol = _mass_tol(E[hh, i].max(), float(np.ptp(S[hh, i])), nT)
                ok = {min(nT, max(m, k_fixed)) for m in _allowed_counts(S[hh, i], rho, tol)}
                assert base[hh, i] in ok, (hh, i, base[hh, i], want_base[hh, i], sorted(ok))
        kh = scope.head_estimate(base[hh], counts)
        assert np.array_equal(keep[hh], np.maximum(base[hh], kh)), hh
    rows = heads * nT
    print(f"  rho={rho} k_fixed={k_fixed}: base counts differing (near the rho crossing) in {off} of {rows} "
          f"rows; k_head {want_kh.tolist()}", flush=True)
    assert off <= max(1, rows // 100)
    assert set(np.unique(M)) <= {0, 1}
    assert np.array_equal(M.sum(axis=2), keep)
    # The chosen tiles: the oracle's top-keep order up to near-ties.
    want = scope.select_rows(S, keep)
    for hh, i, j in np.argwhere(M != want):
        row = np.sort(S[hh, i])[::-1]
        thr = row[keep[hh, i] - 1]
        assert abs(S[hh, i, j] - thr) <= 2 * E[hh, i].max(), (hh, i, j)
    return base, keep


@pytest.mark.parametrize("rho", [0.5, 0.9, 0.99])
def test_hunyuan_inputs(rho):
    wl = make_workload("hunyuan", heads=4)
    nT = oracle.num_tiles(wl.grid, wl.tile)
    k_fixed = math.ceil(nT / 10)   # the page's fixed Top-k ratio 0.1
    print(f"scope hunyuan heads=4 nT={nT} rho={rho} k_fixed={k_fixed}", flush=True)
    _check(wl.grid, wl.tile, wl.q, wl.k, rho, k_fixed)


def test_wan_inputs():
    wl = make_workload("wan", heads=4)
    nT = oracle.num_tiles(wl.grid, wl.tile)
    print(f"scope wan heads=4 nT={nT}", flush=True)
    _check(wl.grid, wl.tile, wl.q, wl.k, 0.8, math.ceil(nT / 10))


@pytest.mark.parametrize("grid,tile,d,dtype", [
    ((4, 8, 8), (1, 4, 4), 64, "f32"),
    ((3, 20, 36), (1, 8, 16), 128, "bf16"),
    ((3, 10, 12), (1, 4, 8), 64, "bf16"),     # 32-token tiles
])
@pytest.mark.parametrize("rho,k_fixed", [(0.3, 0), (0.7, 2), (0.95, 1)])
def test_random_inputs(grid, tile, d, dtype, rho, k_fixed):
    heads, N = 3, int(np.prod(grid))
    rng = np.random.default_rng([21, d, *grid])
    # Scaled inputs: sharper score distributions than unit normals give.
    q = (3 * rng.standard_normal((heads, N, d))).astype(np.float32)
    k = (3 * rng.standard_normal((heads, N, d))).astype(np.float32)
    if dtype == "bf16":
        q = (q.view(np.uint32) >> 16).astype(np.uint16)
        k = (k.view(np.uint32) >> 16).astype(np.uint16)
    print(f"scope grid={grid} tile={tile} d={d} {dtype} rho={rho} k_fixed={k_fixed}", flush=True)
    _check(grid, tile, q, k, rho, k_fixed)


def test_ends():
    """rho <= 0 keeps the fixed count, rho >= 1 every tile; k_fixed = nT
    keeps every tile; ties (all scores equal) go to the lower j."""
    grid, tile, d = (2, 12, 16), (1, 4, 8), 64
    N, nT = int(np.prod(grid)), oracle.num_tiles(grid, tile)
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, N, d)).astype(np.float32)
    q = rng.standard_normal((2, N, d)).astype(np.float32)
    h = sa.sparse_attn_create(2, d, grid, tile, "f32")
    M, base, keep = _gpu(h, q, k, 0.0, 3)
    assert np.all(base == 3) and np.all(keep == 3) and np.all(M.sum(axis=2) == 3)
    M, base, keep = _gpu(h, q, k, 1.0, 0)
    assert np.all(base == nT) and np.all(M == 1)
    M, base, keep = _gpu(h, q, k, 0.5, nT)
    assert np.all(base == nT) and np.all(M == 1)
    z = np.zeros_like(q)                       # every score 0: uniform rows
    M, base, keep = _gpu(h, z, k, 0.5, 0)
    assert np.all(base == math.ceil(0.5 * nT))
    want = np.zeros(nT, np.uint8)
    want[:math.ceil(0.5 * nT)] = 1
    assert all(np.array_equal(M[hh, i], want) for hh in range(2) for i in range(nT))


def test_hilbert_tiles():
    grid, tile, d = (3, 20, 36), (1, 8, 16), 128
    heads, N = 2, int(np.prod(grid))
    rng = np.random.default_rng(31)
    q = (2 * rng.standard_normal((heads, N, d))).astype(np.float32)
    k = (2 * rng.standard_normal((heads, N, d))).astype(np.float32)
    h = sa.sparse_attn_create(heads, d, grid, tile, "f32", order="hilbert")
    ob = torch.empty(sa.sparse_attn_order_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_order(h, ob)
    seq = oracle.hilbert_order(grid)
    # The GPU reads the raster tensors through the order; the oracle sees the
    # tokens in rank order on a 1 x 1 x N grid of 1 x 1 x 128 tiles.
    M, base, keep = _gpu(h, q, k, 0.8, 2)
    S = scope.proxy_scores((1, 1, N), (1, 1, 128), q[:, seq], k[:, seq])
    wb, _, wk = scope.scope_counts(S, oracle.tile_counts((1, 1, N), (1, 1, 128)), 0.8, 2)
    assert np.mean(base == wb) >= 0.99 and np.array_equal(M.sum(axis=2), keep)


def test_rejects_bad_arguments():
    h = sa.sparse_attn_create(2, 64, (2, 8, 8), (1, 4, 4), "f32")
    nT = sa.sparse_attn_layout(h)["tiles"]
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    bm = torch.empty((2, nT, nT), dtype=torch.uint8, device="cuda")
    for rho, kf in [(float("nan"), 0), (float("inf"), 0), (0.5, -1), (0.5, nT + 1)]:
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_select_scope(h, rho, kf, ws, bm)
        assert e.value.status == sa.SPARSE_ATTN_INVALID_ARG
    with pytest.raises(ValueError):
        sa.sparse_attn_select_scope(h, 0.5, 1, ws, bm, base=torch.empty(3, dtype=torch.int32, device="cuda"))

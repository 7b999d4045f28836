"""GPU parity of the Hilbert token order (DFSAttn page, abstract).

In the Hilbert order the tiles are runs of B consecutive Hilbert ranks, so
the expected results come from the oracle run on the tokens taken in rank
order (oracle.hilbert_order) as a 1 x 1 x N grid cut into 1 x 1 x B tiles,
then put back in raster order: the permutation bit-exact, attention within
the usual tolerances, the LSE within its derived bound, the selection
bit-exact up to fp32 near-ties, the pair lists bit-exact."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from workloads import f32_to_bf16_bits, make_workload

from gpu_helpers import as_f64, assert_close, assert_lse_close, dev, host, lse_bound, mass_bound

pytestmark = pytest.mark.gpu


def _rand(shape, seed, dtype):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _handle(heads, d, grid, tile, dtype, pairing="auto"):
    h = sa.sparse_attn_create(heads, d, grid, tile, dtype, order="hilbert", pairing=pairing)
    buf = torch.empty(sa.sparse_attn_order_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_order(h, buf)
    h.order_buf = buf  # keep it alive with the handle
    return h


def _seq_view(grid, tile):
    """(seq, grid1, tile1): rank -> token map and the 1-D grid the oracle
    sees in the Hilbert order."""
    N = int(np.prod(grid))
    return oracle.hilbert_order(grid), (1, 1, N), (1, 1, int(np.prod(tile)))


@pytest.mark.parametrize("grid,tile,d,dtype", [
    ((3, 20, 36), (1, 8, 16), 128, "bf16"),
    ((2, 17, 33), (2, 4, 16), 64, "bf16"),
    ((3, 10, 12), (1, 4, 8), 64, "bf16"),     # 32-token tiles in 128-slot blocks
    ((3, 10, 12), (1, 4, 8), 64, "f32"),
])
def test_permutation_bit_exact(grid, tile, d, dtype):
    heads = 2
    N = int(np.prod(grid))
    h = _handle(heads, d, grid, tile, dtype)
    L = sa.sparse_attn_layout(h)
    B, S, nT = L["tile_volume"], L["slot_stride"], L["tiles"]
    assert B == int(np.prod(tile)) and S == (128 if dtype == "bf16" else B)
    seq = oracle.hilbert_order(grid)
    x = _rand((heads, N, d), 5, dtype)
    # Rank r sits in slot r mod B of tile r // B, row (r // B) S + r mod B.
    r = np.arange(N)
    want = np.zeros((heads, nT * S, d), x.dtype)
    want[:, (r // B) * S + r % B] = x[:, seq]
    xd = dev(x)
    rows = torch.full((heads, nT * S, d), 7, dtype=xd.dtype, device="cuda")
    sa.sparse_attn_permute(h, xd, rows, sa.SPARSE_ATTN_LAYOUT_ROWS)
    back = torch.zeros_like(xd)
    sa.sparse_attn_unpermute(h, rows, back)
    torch.cuda.synchronize()
    assert np.array_equal(host(rows, x), want)
    assert np.array_equal(host(back, x), x)
    if dtype == "bf16":
        cols = torch.full((heads, nT, d, S), 7, dtype=xd.dtype, device="cuda")
        sa.sparse_attn_permute(h, xd, cols, sa.SPARSE_ATTN_LAYOUT_TILE_COLUMNS)
        torch.cuda.synchronize()
        wc = want.reshape(heads, nT, S, d).transpose(0, 1, 3, 2)
        assert np.array_equal(host(cols, x), wc)


def test_calls_need_the_order_buffer():
    h = sa.sparse_attn_create(2, 128, (2, 16, 32), (1, 8, 16), "bf16", order="hilbert")
    x = torch.zeros((2, 2 * 16 * 32, 128), dtype=torch.int16, device="cuda")
    L = sa.sparse_attn_layout(h)
    dst = torch.zeros((2, L["slots"], 128), dtype=torch.int16, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_permute(h, x, dst)
    assert e.value.status == sa.SPARSE_ATTN_NO_ORDER
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_set_order(h, small)
    assert e.value.status == sa.SPARSE_ATTN_WORKSPACE_TOO_SMALL


def _forward(h, q, k, v, M, lse=True, stages=False):
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, bitmap=dev(M))
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.full_like(qd, 0x7FC0 if q.dtype == np.uint16 else 0)
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    L = None
    if stages:
        sa.sparse_attn_permute_inputs(h, qd, kd, vd, ws)
        sa.sparse_attn_attend(h, ws)
        sa.sparse_attn_unpermute_output(h, ws, o)
    else:
        L = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device="cuda") if lse else None
        sa.sparse_attn_forward_lse(h, qd, kd, vd, o, L, ws)
    torch.cuda.synchronize()
    return host(o, q), (L.cpu().numpy() if L is not None else None)


@pytest.mark.parametrize("grid,tile,d,dtype", [
    ((3, 20, 36), (1, 8, 16), 128, "bf16"),   # pair + row kernels
    ((3, 20, 36), (1, 8, 16), 64, "bf16"),
    ((2, 17, 33), (2, 4, 16), 128, "bf16"),
    ((3, 10, 12), (1, 4, 8), 64, "bf16"),     # 32-token tiles in 128-slot blocks
    ((3, 10, 12), (1, 4, 8), 128, "f32"),
])
@pytest.mark.parametrize("pairing", ["auto", "overlap", "all"])  # auto is NONE on these grids
def test_forward_and_lse_match_the_oracle(grid, tile, d, dtype, pairing):
    heads = 3
    N = int(np.prod(grid))
    seq, g1, t1 = _seq_view(grid, tile)
    nT = oracle.num_tiles(g1, t1)
    q, k, v = (_rand((heads, N, d), s, dtype) for s in (11, 12, 13))
    M = (np.random.default_rng(14).random((heads, nT, nT)) < 0.35).astype(np.uint8)
    M[1, nT // 2] = 0
    print(f"hilbert forward grid={grid} tile={tile} d={d} {dtype} pairing={pairing}", flush=True)
    h = _handle(heads, d, grid, tile, dtype, pairing)
    o, lse = _forward(h, q, k, v, M)
    staged, _ = _forward(h, q, k, v, M, stages=True)
    assert np.array_equal(o, staged)
    qs, ks, vs = q[:, seq], k[:, seq], v[:, seq]
    want_s, lse_s = oracle.attention(g1, t1, qs, ks, vs, M, lse=True)
    want = np.empty_like(want_s)
    want[:, seq] = want_s
    assert_close(as_f64(o), want, dtype, "hilbert o")
    want_lse = np.empty_like(lse_s)
    want_lse[:, seq] = lse_s
    counts = oracle.tile_counts(g1, t1)
    kept_s = (M.astype(np.int64) @ counts)[:, np.arange(N) // t1[2]]
    kept = np.empty_like(kept_s)
    kept[:, seq] = kept_s
    kmax = np.array([np.linalg.norm(as_f64(k[i]), axis=-1).max() for i in range(heads)])
    bound = lse_bound(as_f64(q).reshape(-1, d), np.repeat(kmax, N), kept.reshape(-1), d,
                      1.0 / np.sqrt(d), dtype, want_lse.reshape(-1))
    assert_lse_close(lse.reshape(-1).astype(np.float64), want_lse.reshape(-1), bound, "hilbert")


def test_selection_on_hilbert_tiles():
    grid, tile, d = (3, 20, 36), (1, 8, 16), 128
    heads = 3
    N = int(np.prod(grid))
    seq, g1, t1 = _seq_view(grid, tile)
    nT = oracle.num_tiles(g1, t1)
    q, k = (_rand((heads, N, d), s, "bf16") for s in (21, 22))
    kh = [1, nT // 3, nT - 1]
    h = _handle(heads, d, grid, tile, "bf16")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    qd, kd = dev(q), dev(k)
    sa.sparse_attn_permute_inputs(h, qd, kd, kd, ws)
    bm = torch.empty((heads, nT, nT), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_select_topk(h, kh, ws, bm)
    torch.cuda.synchronize()
    got = bm.cpu().numpy()
    want = oracle.select_topk(g1, t1, q[:, seq], k[:, seq], kh)
    for hh in range(heads):
        assert (got[hh].sum(axis=1) == kh[hh]).all()
    diff = np.argwhere(got != want)
    if len(diff):  # only fp32 near-ties may differ
        S = np.stack([oracle.tile_means(g1, t1, q[i, seq]) @ oracle.tile_means(g1, t1, k[i, seq]).T
                      for i in range(heads)]) / np.sqrt(d)
        for hh, i, j in diff:
            thr = np.sort(S[hh, i])[::-1][kh[hh] - 1]
            assert abs(S[hh, i, j] - thr) <= 1e-5 * max(1.0, abs(thr))


def test_pair_lists_on_hilbert_tiles():
    from test_gpu_pair_lists import _check
    grid, tile = (3, 20, 36), (1, 8, 16)
    seq, g1, t1 = _seq_view(grid, tile)
    nT = oracle.num_tiles(g1, t1)
    M = (np.random.default_rng(31).random((3, nT, nT)) < 0.3).astype(np.uint8)
    h = _handle(3, 128, grid, tile, "bf16")
    _check(h, M, g1, t1, bitmap=M)


def test_full_size_wan_shape_sampled():
    """Wan-shaped inputs at full size (40 heads x 75,600 tokens) with top-k
    masks chosen on the Hilbert tiles by the GPU selection; sampled query
    rows against the oracle under the same masks."""
    wl = make_workload("wan", masks_only=False)
    grid, tile, d = wl.grid, wl.tile, wl.head_dim
    seq, g1, t1 = _seq_view(grid, tile)
    nT = oracle.num_tiles(g1, t1)
    heads = wl.heads
    kh = [max(1, round(wl.info["tile_density"] * nT))] * heads
    print(f"hilbert wan full: nT={nT} k={kh[0]}", flush=True)
    h = _handle(heads, d, grid, tile, "bf16")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    sa.sparse_attn_permute_inputs(h, q, k, v, ws)
    bm = torch.empty((heads, nT, nT), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_select_topk(h, kh, ws, bm)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, bitmap=bm)
    o = torch.empty_like(q)
    sa.sparse_attn_forward(h, q, k, v, o, ws)
    torch.cuda.synchronize()
    M = bm.cpu().numpy()
    N = wl.config.tokens
    rank = np.empty(N, dtype=np.int64)
    rank[seq] = np.arange(N)
    rng = np.random.default_rng(5)
    toks = rng.choice(N, size=16, replace=False)
    rows_raster = np.concatenate([hh * N + toks for hh in range(heads)])
    rows_seq = np.concatenate([hh * N + rank[toks] for hh in range(heads)])
    want = oracle.attention_rows(g1, t1, wl.q[:, seq], wl.k[:, seq], wl.v[:, seq], M, rows_seq)
    got = as_f64(host(o, wl.q).reshape(-1, d)[rows_raster])
    assert_close(got, want, "bf16", f"hilbert wan ({len(rows_raster)} sampled rows)")


def test_tile_mass_on_hilbert_tiles():
    """The full-attention tile mass on Hilbert tiles equals the oracle's on
    the rank-ordered 1-D grid, within the mass bound."""
    grid, tile, d, heads = (3, 20, 36), (1, 8, 16), 128, 2
    N = int(np.prod(grid))
    seq, g1, t1 = _seq_view(grid, tile)
    q, k = (_rand((heads, N, d), s, "bf16") for s in (21, 22))
    h = _handle(heads, d, grid, tile, "bf16")
    nT = sa.sparse_attn_layout(h)["tiles"]
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    mass = torch.full((heads, nT, nT), -1.0, dtype=torch.float32, device="cuda")
    print(f"hilbert tile mass grid={grid} tiles={nT}", flush=True)
    sa.sparse_attn_tile_mass(h, dev(q), dev(k), ws, mass)
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    want = oracle.tile_mass(g1, t1, q[:, seq], k[:, seq])
    err = np.abs(got - want)
    bound = mass_bound(q, k, want, N)
    print(f"  max abs {err.max():.3e}, max err/bound {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)

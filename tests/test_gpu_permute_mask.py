"""GPU parity of the tile-major permutation and the mask compiler: bit-exact
against the oracle's slot maps and index lists."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from workloads import make_workload

from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

GRIDS = [
    ((4, 8, 8), (1, 4, 4), 64, "f32"),
    ((8, 30, 40), (1, 8, 16), 128, "bf16"),
    ((3, 20, 36), (1, 8, 16), 128, "bf16"),
    ((3, 20, 36), (1, 8, 16), 64, "bf16"),
    ((3, 20, 36), (1, 4, 8), 128, "bf16"),    # 32-token tiles in 128-slot blocks
    ((1, 5, 7), (1, 8, 16), 128, "bf16"),
    ((3, 10, 12), (1, 4, 8), 64, "f32"),
    ((5, 3, 3), (2, 3, 3), 128, "f32"),
    ((21, 45, 80), (1, 8, 16), 128, "bf16"),
]


def _random_bits(shape, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "bf16":
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return rng.standard_normal(shape, dtype=np.float32)


@pytest.mark.parametrize("grid,tile,d,dtype", GRIDS)
def test_permute_and_unpermute_bit_exact(grid, tile, d, dtype):
    heads = 3
    N = int(np.prod(grid))
    B = int(np.prod(tile))
    nT = oracle.num_tiles(grid, tile)
    print(f"permute grid={grid} tile={tile} d={d} {dtype}", flush=True)
    x = _random_bits((heads, N, d), dtype, 1)
    h = sa.sparse_attn_create(heads, d, grid, tile, dtype)
    L = sa.sparse_attn_layout(h)
    # bf16 tiles take 128 slots whatever their volume (matrix-core blocks),
    # fp32 tiles B.
    S = 128 if dtype == "bf16" else B
    assert L["tiles"] == nT and L["tile_volume"] == B and L["slot_stride"] == S
    assert L["slots"] == nT * S and L["tokens"] == N
    # The oracle's slot map has B slots per tile; slot s of tile t moves to
    # t S + s.
    perm, pos = oracle.perm(grid, tile)
    want = np.zeros((heads, nT, S, d), dtype=x.dtype)
    pm = perm.reshape(nT, B)
    real = pm >= 0
    want[:, :, :B][:, real] = x[:, pm[real]]
    want = want.reshape(heads, nT * S, d)

    xd = dev(x)
    rows = torch.full((heads, nT * S, d), 7, dtype=xd.dtype, device="cuda")  # pads must be zeroed
    sa.sparse_attn_permute(h, xd, rows, sa.SPARSE_ATTN_LAYOUT_ROWS)
    got = host(rows, x)
    assert np.array_equal(got, want)

    back = torch.full_like(xd, 3)
    sa.sparse_attn_unpermute(h, rows, back)
    assert np.array_equal(host(back, x), x)

    if dtype == "bf16":
        cols = torch.full((heads, nT, d, S), 5, dtype=xd.dtype, device="cuda")
        sa.sparse_attn_permute(h, xd, cols, sa.SPARSE_ATTN_LAYOUT_TILE_COLUMNS)
        want_cols = want.reshape(heads, nT, S, d).transpose(0, 1, 3, 2)
        assert np.array_equal(host(cols, x), want_cols)


def _gpu_csr(h, R, nnz_cap, bitmap=None, groups=None, gph=None, max_nnz=0):
    mb = torch.empty(sa.sparse_attn_mask_bytes(h, max_nnz), dtype=torch.uint8, device="cuda")
    if bitmap is not None:
        sa.sparse_attn_set_mask(h, mb, bitmap=dev(bitmap), max_nnz=max_nnz)
    else:
        sa.sparse_attn_set_mask(h, mb, groups=groups, groups_per_head=gph, max_nnz=max_nnz)
    row_ptr = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    cols = torch.full((max(nnz_cap, 1),), -7, dtype=torch.int32, device="cuda")
    order = torch.empty(R, dtype=torch.int32, device="cuda")
    sa.sparse_attn_read_index_lists(h, row_ptr, cols, order)
    nnz, ovf = sa.sparse_attn_mask_info(h)
    return row_ptr.cpu().numpy(), cols.cpu().numpy(), order.cpu().numpy(), nnz, ovf


def _check_against_oracle(h, M, **mask):
    heads, nT, _ = M.shape
    R = heads * nT
    row_ptr, cols, order = oracle.csr(M)
    g_rp, g_cols, g_order, nnz, ovf = _gpu_csr(h, R, len(cols), **mask)
    assert nnz == len(cols) and not ovf
    assert np.array_equal(g_rp, row_ptr)
    assert np.array_equal(g_cols[:len(cols)], cols)
    assert np.array_equal(g_order, order)


@pytest.mark.parametrize("name", ["tiny", "small", "wan", "hunyuan", "long"])
def test_workload_masks_bit_exact(name):
    wl = make_workload(name, heads=4 if name == "hunyuan" else None, masks_only=True)
    print(f"mask {name} heads={wl.heads} kind={wl.mask_kind}", flush=True)
    M = oracle.mask_of(wl)
    h = sa.sparse_attn_create(wl.heads, wl.head_dim, wl.grid, wl.tile, wl.dtype)
    if wl.mask_kind == "windows":
        _check_against_oracle(h, M, groups=wl.groups, gph=wl.groups_per_head)
    # the bitmap path on the same mask
    _check_against_oracle(h, M, bitmap=M)


def _random_specs(rng, heads, tgrid):
    nt, ny, nx = tgrid
    groups, gph = [], []
    for _ in range(heads):
        n = int(rng.integers(1, 4))
        cuts = np.sort(rng.choice(np.arange(1, nt + 3), size=n, replace=False))
        lo = 0  # groups are sorted and disjoint: [0, c0 - 1], [c0, c1 - 1], ...
        for gi in range(n):
            last = gi + 1 == n
            hi = -1 if last and rng.random() < 0.5 else int(cuts[gi]) - 1
            r = rng.integers(-1, max(ny, nx) + 1, size=4).tolist()
            groups.append([lo, hi, *r])
            lo = hi + 1
        gph.append(n)
    return np.array(groups, np.int32), np.array(gph, np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_random_window_specs_bit_exact(seed):
    rng = np.random.default_rng(900 + seed)
    grid, tile = [((5, 30, 40), (1, 8, 16)), ((7, 13, 11), (2, 3, 2)), ((9, 20, 20), (1, 4, 4))][seed % 3]
    tgrid = tuple(-(-g // t) for g, t in zip(grid, tile))
    heads = 5
    groups, gph = _random_specs(rng, heads, tgrid)
    print(f"random spec seed={seed} grid={grid} groups={len(groups)}", flush=True)
    M = oracle.mask_from_windows(grid, tile, groups, gph)
    h = sa.sparse_attn_create(heads, 64, grid, tile, "f32")
    _check_against_oracle(h, M, groups=groups, gph=gph)


@pytest.mark.parametrize("p", [0.0, 0.05, 0.5, 1.0])
def test_random_bitmaps_bit_exact(p):
    rng = np.random.default_rng(int(p * 100) + 5)
    grid, tile = (6, 24, 40), (1, 8, 8)
    nT = oracle.num_tiles(grid, tile)
    M = ((rng.random((3, nT, nT)) < p) * rng.integers(1, 256, size=(3, nT, nT))).astype(np.uint8)
    M[1, 3, :] = 0  # an empty row
    h = sa.sparse_attn_create(3, 64, grid, tile, "f32")
    _check_against_oracle(h, M, bitmap=M)


def test_index_list_overflow_is_reported_and_truncated():
    wl = make_workload("small", masks_only=True)
    M = oracle.mask_of(wl)
    row_ptr, cols, order = oracle.csr(M)
    cap = len(cols) // 2
    h = sa.sparse_attn_create(wl.heads, 128, wl.grid, wl.tile, "bf16")
    g_rp, g_cols, g_order, nnz, ovf = _gpu_csr(h, wl.heads * 96, cap, groups=wl.groups,
                                              gph=wl.groups_per_head, max_nnz=cap)
    assert ovf and nnz == len(cols)
    assert np.array_equal(g_rp, row_ptr) and np.array_equal(g_cols[:cap], cols[:cap])

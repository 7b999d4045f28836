"""GPU parity of the query-tile pair lists that the matrix-core kernels walk:
bit-exact against lists built here from the oracle's mask.

The pairing, the packed entry and the acceptance rule are the library's own
work split (the pages define only the per-tile mask); the expected lists are
derived from the oracle's mask and tile sizes alone, by the rule the header
documents: tiles (2c, 2c + 1) along the pair axis form pair c; the list of a
pair the pair kernel serves is the ascending union of its tiles' rows, each
entry j | c_j << 16 | keep bits << 24; under the OVERLAP pairing a pair is
served when 10 |union| <= 7 (|row 1| + |row 2|), under ALL always, under
NONE never (AUTO: NONE for layouts of at most 1024 pairs over all heads,
else OVERLAP); a pair not served has an empty list; the work order sorts
pairs by decreasing list length, ties by pair id."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from workloads import make_workload

from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _tile_pairs(L):
    """(t1, t2) per pair, raster over the pair grid; t2 = -1 when alone."""
    nt, ny, nx = L["tile_grid"]
    pn = L["pair_grid"]
    ax = L["pair_axis"]
    out = []
    for a in range(pn[0]):
        for b in range(pn[1]):
            for e in range(pn[2]):
                c1 = [a, b, e]
                c2 = None
                if ax >= 0:
                    c1[ax] *= 2
                    c2 = list(c1)
                    c2[ax] += 1
                    if c2[ax] >= (nt, ny, nx)[ax]:
                        c2 = None
                t1 = (c1[0] * ny + c1[1]) * nx + c1[2]
                t2 = -1 if c2 is None else (c2[0] * ny + c2[1]) * nx + c2[2]
                out.append((t1, t2))
    return out


def _expected(M, L, counts, mode):
    heads, nT, _ = M.shape
    pairs = _tile_pairs(L)
    P = len(pairs)
    want_pairing = mode if mode != sa.SPARSE_ATTN_PAIRING_AUTO else (
        sa.SPARSE_ATTN_PAIRING_NONE if heads * P <= 1024 else sa.SPARSE_ATTN_PAIRING_OVERLAP)
    assert L["pairing"] == want_pairing
    lens, flags, lists = [], [], []
    for h in range(heads):
        for t1, t2 in pairs:
            k1 = M[h, t1].astype(bool)
            k2 = M[h, t2].astype(bool) if t2 >= 0 else np.zeros(nT, bool)
            bits = k1.astype(np.int64) | (k2.astype(np.int64) << 1)
            j = np.nonzero(bits)[0]
            if want_pairing == sa.SPARSE_ATTN_PAIRING_ALL:
                served = True
            elif want_pairing == sa.SPARSE_ATTN_PAIRING_NONE:
                served = False
            else:
                served = 10 * len(j) <= 7 * (int(k1.sum()) + int(k2.sum()))
            flags.append(int(served))
            if served:
                lists.append(j | (counts[j].astype(np.int64) << 16) | (bits[j] << 24))
                lens.append(len(j))
            else:
                lists.append(np.zeros(0, np.int64))
                lens.append(0)
    lens = np.array(lens, np.int64)
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cols = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
    order = np.array(sorted(range(heads * P), key=lambda r: (-lens[r], r)), np.int32)
    return row_ptr, cols, order, np.array(flags, np.int32)


def _check(h, M, grid, tile, mode=0, **mask):
    L = sa.sparse_attn_layout(h)
    counts = oracle.tile_counts(grid, tile)
    row_ptr, cols, order, flags = _expected(M, L, counts, mode)
    heads = M.shape[0]
    P = heads * L["pairs"]
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    if "bitmap" in mask:
        sa.sparse_attn_set_mask(h, mb, bitmap=dev(mask["bitmap"]))
    else:
        sa.sparse_attn_set_mask(h, mb, groups=mask["groups"], groups_per_head=mask["gph"])
    g_rp = torch.empty(P + 1, dtype=torch.int32, device="cuda")
    g_cols = torch.full((max(len(cols), 1),), -7, dtype=torch.int32, device="cuda")
    g_order = torch.empty(P, dtype=torch.int32, device="cuda")
    g_flag = torch.empty(P, dtype=torch.int32, device="cuda")
    sa.sparse_attn_read_pair_lists(h, g_rp, g_cols, g_order, g_flag)
    torch.cuda.synchronize()
    assert np.array_equal(g_flag.cpu().numpy(), flags)
    assert np.array_equal(g_rp.cpu().numpy(), row_ptr)
    assert np.array_equal(g_cols.cpu().numpy()[:len(cols)], cols)
    assert np.array_equal(g_order.cpu().numpy(), order)
    return flags


@pytest.mark.parametrize("name", ["small", "wan", "hunyuan", "long"])
def test_workload_pair_lists_bit_exact(name):
    heads = 4 if name != "small" else None
    wl = make_workload(name, heads=heads, masks_only=True)
    print(f"pair lists {name} heads={wl.heads} grid={wl.grid}", flush=True)
    M = oracle.mask_of(wl)
    # OVERLAP, the split AUTO takes at full size (Small alone would run as NONE)
    h = sa.sparse_attn_create(wl.heads, 128, wl.grid, wl.tile, "bf16", pairing="overlap")
    mode = sa.SPARSE_ATTN_PAIRING_OVERLAP
    if wl.mask_kind == "bitmap":
        flags = _check(h, M, wl.grid, wl.tile, mode, bitmap=wl.bitmap)
    else:
        flags = _check(h, M, wl.grid, wl.tile, mode, groups=wl.groups, gph=wl.groups_per_head)
    print(f"  pairs served by the pair kernel: {flags.mean():.3f}", flush=True)


# Tile grids that make every pair axis appear, with a tile left alone at an
# odd edge: y (ny even), t (ny odd, nt even), x (ny, nt odd, nx even), and
# y with odd extent everywhere (singles).
PAIR_GRIDS = [
    ((3, 32, 32), (1, 8, 16)),   # tile grid 3 x 4 x 2 -> y
    ((4, 24, 32), (1, 8, 16)),   # 4 x 3 x 2 -> t
    ((3, 24, 64), (1, 8, 16)),   # 3 x 3 x 4 -> x
    ((3, 40, 48), (1, 8, 16)),   # 3 x 5 x 3 -> y, last tile row alone
    ((1, 8, 16), (1, 8, 16)),    # one tile -> no pairing
]


@pytest.mark.parametrize("grid,tile", PAIR_GRIDS)
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("pairing", ["auto", "overlap", "all"])  # auto is NONE on these grids
def test_random_bitmap_pair_lists_bit_exact(grid, tile, density, pairing):
    heads = 3
    nT = oracle.num_tiles(grid, tile)
    rng = np.random.default_rng([7, int(density * 10), *grid])
    M = (rng.random((heads, nT, nT)) < density).astype(np.uint8)
    print(f"pair lists grid={grid} density={density} pairing={pairing}", flush=True)
    h = sa.sparse_attn_create(heads, 128, grid, tile, "bf16", pairing=pairing)
    _check(h, M, grid, tile, mode=sa._PAIRINGS[pairing], bitmap=M)


def test_pair_lists_need_the_matrix_core_kernel():
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    z = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_read_pair_lists(h, z, z, z, z)
    assert e.value.status == sa.SPARSE_ATTN_UNSUPPORTED

"""The C-ABI library: exported symbols and host-side argument checks.

These run without a GPU: every call here fails validation (or is host-only)
before the library touches the device.  Device pointers are fake, aligned,
non-null integers that are never dereferenced.
"""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def sa():
    lib = os.path.join(ROOT, "block_sparse_attention_major_amd", "libsparse_attn.so")
    if not os.path.exists(lib):
        from block_sparse_attention_major_amd import build as b
        b.build()
    import block_sparse_attention_major_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["sparse_attn_create", "sparse_attn_forward", "sparse_attn_destroy",
              "sparse_attn_set_mask", "sparse_attn_mask_bytes", "sparse_attn_workspace_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol(sa):
    lib = ctypes.CDLL(sa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(sa.EXPORTED) == _declared()


def test_create_and_layout(sa):
    h = sa.sparse_attn_create(40, 128, (21, 45, 80), (1, 8, 16), "bf16")
    L = sa.sparse_attn_layout(h)
    assert L["tokens"] == 75600 and L["tiles"] == 630 and L["tile_grid"] == [21, 6, 5]
    assert L["tile_volume"] == 128 and L["slot_stride"] == 128 and L["slots"] == 80640
    assert L["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_BF16
    assert L["v_layout"] == sa.SPARSE_ATTN_LAYOUT_TILE_COLUMNS
    per = 40 * 80640 * 128 * 2
    assert L["ws_bytes"] == sa.sparse_attn_workspace_bytes(h) == 4 * per
    assert L["ws_offset_k"] == per and L["ws_offset_o"] == 3 * per
    # The matrix-core kernel keeps two index lists (query-tile rows and
    # query-tile pairs) of max_nnz entries each.
    full = sa.sparse_attn_mask_bytes(h)
    assert full >= 2 * 40 * 630 * 630 * 4
    shrink = full - sa.sparse_attn_mask_bytes(h, 1000)
    assert abs(shrink - 8 * (40 * 630 * 630 - 1000)) < 256
    sa.sparse_attn_destroy(h)
    tiny = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    L = sa.sparse_attn_layout(tiny)
    assert L["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_F32 and L["pairing"] == -1
    assert L["v_layout"] == sa.SPARSE_ATTN_LAYOUT_ROWS
    assert L["tile_volume"] == L["slot_stride"] == 16 and L["slots"] == 16 * 16
    full = sa.sparse_attn_mask_bytes(tiny)
    assert sa.sparse_attn_mask_bytes(tiny, 100) == full - 4 * (2 * 16 * 16 - 100)
    vec = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32", vector_alu=True)
    assert sa.sparse_attn_layout(vec)["kernel"] == sa.SPARSE_ATTN_KERNEL_GENERIC
    # fp32 layouts whose tile-major rows of one head reach 2^31 bytes run on
    # the vector ALUs (the fp32 matrix-core kernel addresses a head with 32
    # bits): 33,000 tiles of 128 tokens, d = 128, are 2.16 GB per head.
    big = sa.sparse_attn_create(1, 128, (1, 24, 16 * 11000), (1, 8, 16), "f32")
    assert sa.sparse_attn_layout(big)["kernel"] == sa.SPARSE_ATTN_KERNEL_GENERIC
    mid = sa.sparse_attn_create(1, 128, (1, 24, 16 * 5000), (1, 8, 16), "f32")
    assert sa.sparse_attn_layout(mid)["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_F32


def test_small_bf16_tiles_take_matrix_core_blocks(sa):
    # bf16 tiles of any volume run on the matrix cores in blocks of 128
    # slots; vector_alu keeps them on the vector ALUs with B slots per tile.
    h = sa.sparse_attn_create(3, 64, (3, 10, 12), (1, 4, 8), "bf16")
    L = sa.sparse_attn_layout(h)
    assert L["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_BF16
    assert L["v_layout"] == sa.SPARSE_ATTN_LAYOUT_TILE_COLUMNS
    assert L["tiles"] == 3 * 3 * 2 and L["tile_volume"] == 32 and L["slot_stride"] == 128
    assert L["slots"] == 18 * 128 and L["ws_bytes"] == 4 * 3 * 18 * 128 * 64 * 2
    v = sa.sparse_attn_create(3, 64, (3, 10, 12), (1, 4, 8), "bf16", vector_alu=True)
    L = sa.sparse_attn_layout(v)
    assert L["kernel"] == sa.SPARSE_ATTN_KERNEL_GENERIC and L["v_layout"] == sa.SPARSE_ATTN_LAYOUT_ROWS
    assert L["tile_volume"] == L["slot_stride"] == 32 and L["slots"] == 18 * 32
    # the Hilbert order: 1 x 1 x B tiles, still 128 slots each
    hb = sa.sparse_attn_create(2, 128, (2, 16, 32), (1, 4, 16), "bf16", order="hilbert")
    L = sa.sparse_attn_layout(hb)
    assert L["tile_volume"] == 64 and L["slot_stride"] == 128 and L["slots"] == 16 * 128


@pytest.mark.parametrize("grid,axis,pgrid", [
    ((21, 45, 80), 1, [21, 3, 5]),   # tile grid 21 x 6 x 5: y even
    ((4, 24, 32), 0, [2, 3, 2]),     # 4 x 3 x 2: y odd, t even
    ((3, 24, 64), 2, [3, 3, 2]),     # 3 x 3 x 4: only x even
    ((3, 40, 48), 1, [3, 3, 3]),     # 3 x 5 x 3: all odd -> y, last tile row alone
    ((1, 8, 16), -1, [1, 1, 1]),     # one tile: no pairing
])
def test_pair_axis_choice(sa, grid, axis, pgrid):
    h = sa.sparse_attn_create(2, 128, grid, (1, 8, 16), "bf16")
    L = sa.sparse_attn_layout(h)
    assert L["pair_axis"] == axis and L["pair_grid"] == pgrid
    assert L["pairs"] == pgrid[0] * pgrid[1] * pgrid[2]
    sa.sparse_attn_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(heads=0), 1), (dict(grid=(0, 8, 8)), 1), (dict(tile=(1, 0, 4)), 1),
    (dict(dtype=7), 1), (dict(softmax_scale=-1.0), 1), (dict(softmax_scale=float("inf")), 1),
    (dict(head_dim=96), 2), (dict(tile=(2, 8, 16)), 2), (dict(grid=(400, 64, 64), tile=(1, 1, 1)), 2),
    (dict(order=5), 1), (dict(grid=(4, 8, 1 << 22), order=1), 2),
])
def test_create_rejects(sa, kw, code):
    args = dict(heads=2, head_dim=64, grid=(4, 8, 8), tile=(1, 4, 4), dtype="f32", softmax_scale=0.0)
    args.update(kw)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_create(**args)
    assert e.value.status == code
    assert sa.sparse_attn_last_error(None)


def test_largest_tile_count(sa):
    """heads * tiles^2 must stay below 2^31 (32-bit index lists, tile ids
    below 2^16): 46,340 tiles of one head are accepted, 46,341 are not."""
    h = sa.sparse_attn_create(1, 128, (331, 80, 224), (1, 8, 16), "bf16")
    L = sa.sparse_attn_layout(h)
    assert L["tiles"] == 46340 and L["tokens"] == 5931520 and L["slots"] == 5931520
    assert 46340 ** 2 < 2 ** 31 <= 46341 ** 2
    sa.sparse_attn_destroy(h)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_create(1, 128, (1, 24, 16 * 15447), (1, 8, 16), "bf16")  # 3 x 15,447 tiles
    assert e.value.status == sa.SPARSE_ATTN_UNSUPPORTED
    with pytest.raises(sa.SparseAttnError):
        sa.sparse_attn_create(2, 128, (331, 80, 224), (1, 8, 16), "bf16")  # 2 heads of 46,340


FAKE = 1 << 40  # aligned, never dereferenced


def _ws(sa, h):
    return sa.sparse_attn_workspace_bytes(h)


def test_forward_before_set_mask(sa):
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    st = sa._lib.sparse_attn_forward(h.ptr, FAKE, FAKE + 2**30, FAKE + 2**31, FAKE + 2**32,
                                     FAKE + 2**33, _ws(sa, h), None)
    assert st == sa.SPARSE_ATTN_NO_MASK
    st = sa._lib.sparse_attn_attend(h.ptr, FAKE, _ws(sa, h), None)
    assert st == sa.SPARSE_ATTN_NO_MASK


def test_forward_argument_checks(sa):
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    f = sa._lib.sparse_attn_forward
    ws = FAKE + 2**33
    assert f(h.ptr, None, FAKE, FAKE, FAKE, ws, _ws(sa, h), None) == sa.SPARSE_ATTN_INVALID_ARG
    assert f(h.ptr, FAKE + 4, FAKE, FAKE, FAKE, ws, _ws(sa, h), None) == sa.SPARSE_ATTN_INVALID_ARG
    assert f(h.ptr, FAKE, FAKE, FAKE, FAKE, ws, _ws(sa, h) - 1, None) == sa.SPARSE_ATTN_WORKSPACE_TOO_SMALL
    assert "workspace" in sa.sparse_attn_last_error(h)
    assert f(None, FAKE, FAKE, FAKE, FAKE, ws, 0, None) == sa.SPARSE_ATTN_INVALID_ARG


def _set_mask_raw(sa, h, groups, gph, nbytes=None):
    g = np.ascontiguousarray(groups, dtype=np.int32).reshape(-1, 6)
    gph = np.ascontiguousarray(gph, dtype=np.int32)
    m = sa.sparse_attn_mask()
    m.kind = sa.SPARSE_ATTN_MASK_DUAL_WINDOW
    m.groups = g.ctypes.data
    m.groups_per_head = gph.ctypes.data
    m.max_nnz = 0
    n = sa.sparse_attn_mask_bytes(h) if nbytes is None else nbytes
    return sa._lib.sparse_attn_set_mask(h.ptr, ctypes.byref(m), FAKE, n, None)


@pytest.mark.parametrize("groups,gph", [
    ([[0, 0, 1, 1, 1, 1]], [0, 1]),                              # no groups for head 0
    ([[0, 0, 1, 1, 1, 1]] * 9 + [[0, 0, 1, 1, 1, 1]], [9, 1]),   # too many groups
    ([[1, 0, 1, 1, 1, 1], [0, 0, 1, 1, 1, 1]], [1, 1]),          # dt_hi < dt_lo
    ([[-1, 0, 1, 1, 1, 1], [0, 0, 1, 1, 1, 1]], [1, 1]),         # negative dt_lo
    ([[0, -1, 1, 1, 1, 1], [3, 4, 1, 1, 1, 1], [0, 0, 0, 0, 0, 0]], [2, 1]),  # unbounded not last
    ([[0, 2, 1, 1, 1, 1], [2, 3, 1, 1, 1, 1], [0, 0, 0, 0, 0, 0]], [2, 1]),   # overlapping
    ([[0, 0, -2, 1, 1, 1], [0, 0, 1, 1, 1, 1]], [1, 1]),         # extent below -1
    ([[0, -2, 1, 1, 1, 1], [0, 0, 1, 1, 1, 1]], [1, 1]),         # dt_hi below -1
])
def test_set_mask_rejects_malformed_specs(sa, groups, gph):
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    assert _set_mask_raw(sa, h, groups, gph) == sa.SPARSE_ATTN_BAD_MASK
    assert sa.sparse_attn_last_error(h)


def test_set_mask_buffer_and_kind_checks(sa):
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    ok = [[0, 0, 1, 1, 1, 1]] * 2
    assert _set_mask_raw(sa, h, ok, [1, 1], nbytes=100) == sa.SPARSE_ATTN_WORKSPACE_TOO_SMALL
    m = sa.sparse_attn_mask()
    m.kind = 5
    assert sa._lib.sparse_attn_set_mask(h.ptr, ctypes.byref(m), FAKE, 1 << 20, None) == sa.SPARSE_ATTN_BAD_MASK
    m.kind = sa.SPARSE_ATTN_MASK_BITMAP
    m.bitmap = None
    assert sa._lib.sparse_attn_set_mask(h.ptr, ctypes.byref(m), FAKE, 1 << 20, None) == sa.SPARSE_ATTN_INVALID_ARG
    assert sa._lib.sparse_attn_set_mask(h.ptr, None, FAKE, 1 << 20, None) == sa.SPARSE_ATTN_INVALID_ARG


def test_permute_hook_checks(sa):
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    p = sa._lib.sparse_attn_permute
    assert p(h.ptr, FAKE, FAKE + 2**30, 9, None) == sa.SPARSE_ATTN_INVALID_ARG
    assert p(h.ptr, FAKE, FAKE + 2**30, sa.SPARSE_ATTN_LAYOUT_TILE_COLUMNS, None) == sa.SPARSE_ATTN_UNSUPPORTED
    assert p(h.ptr, None, FAKE, 0, None) == sa.SPARSE_ATTN_INVALID_ARG
    r = sa._lib.sparse_attn_read_index_lists
    assert r(h.ptr, FAKE, FAKE, 10, FAKE, None) == sa.SPARSE_ATTN_NO_MASK


def test_hilbert_layout(sa):
    """Hilbert order: runs of B ranks form a 1 x 1 x nT tile grid, the last
    tile clipped; the order buffer holds one int32 per token."""
    h = sa.sparse_attn_create(2, 128, (3, 20, 36), (1, 8, 16), "bf16", order="hilbert")
    L = sa.sparse_attn_layout(h)
    N = 3 * 20 * 36
    assert L["order"] == sa.SPARSE_ATTN_ORDER_HILBERT and L["tokens"] == N
    assert L["tiles"] == -(-N // 128) and L["tile_grid"] == [1, 1, L["tiles"]]
    assert L["slots"] == L["tiles"] * 128 and L["pair_axis"] == 2
    assert sa.sparse_attn_order_bytes(h) == 4 * N
    t = sa.sparse_attn_create(2, 128, (3, 20, 36), (1, 8, 16), "bf16")
    assert sa.sparse_attn_layout(t)["order"] == sa.SPARSE_ATTN_ORDER_TILES
    assert sa.sparse_attn_order_bytes(t) == 0
    assert sa._lib.sparse_attn_set_order(t.ptr, None, 0, None) == 0  # nothing to do


def test_hilbert_calls_need_the_order(sa):
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32", order="hilbert")
    st = sa._lib.sparse_attn_forward(h.ptr, FAKE, FAKE + 2**30, FAKE + 2**31, FAKE + 2**32,
                                     FAKE + 2**33, _ws(sa, h), None)
    assert st == sa.SPARSE_ATTN_NO_ORDER
    assert sa._lib.sparse_attn_permute(h.ptr, FAKE, FAKE + 2**30, 0, None) == sa.SPARSE_ATTN_NO_ORDER
    assert sa._lib.sparse_attn_set_order(h.ptr, FAKE + 8, 1 << 20, None) == sa.SPARSE_ATTN_INVALID_ARG
    assert sa._lib.sparse_attn_set_order(h.ptr, FAKE, 16, None) == sa.SPARSE_ATTN_WORKSPACE_TOO_SMALL


def test_status_strings(sa):
    assert sa.sparse_attn_status_string(0) == "ok"
    assert "mask" in sa.sparse_attn_status_string(sa.SPARSE_ATTN_NO_MASK)
    assert "Hilbert" in sa.sparse_attn_status_string(sa.SPARSE_ATTN_NO_ORDER)
    assert sa.sparse_attn_status_string(99) == "unknown status"


def test_binding_refuses_mis_sized_host_arrays(sa):
    """Host arrays the C side reads or writes per head are checked against
    the handle before the call (no device needed: the checks come first)."""
    h = sa.sparse_attn_create(3, 128, (2, 16, 32), (1, 8, 16), "bf16")
    nT = sa.sparse_attn_layout(h)["tiles"]
    mass = np.zeros((3, nT, nT), np.float32)
    groups = np.array([(0, 0, 0, 0, 0, 0)] * 3, np.int32)
    with pytest.raises(ValueError):  # groups_per_head for 2 of 3 heads
        sa.sparse_attn_search_windows(h, mass, groups[:2], np.ones(2, np.int32), 0.9)
    with pytest.raises(ValueError):  # rows != sum(groups_per_head)
        sa.sparse_attn_search_windows(h, mass, groups[:2], np.ones(3, np.int32), 0.9)
    with pytest.raises(ValueError):  # mass of 2 heads
        sa.sparse_attn_search_windows(h, mass[:2], groups, np.ones(3, np.int32), 0.9)
    with pytest.raises(ValueError):
        sa.sparse_attn_set_mask(h, None, groups=groups, groups_per_head=np.ones(4, np.int32))
    with pytest.raises(ValueError):
        sa.sparse_attn_select_topk(h, [1, 2], None, None)


def test_noalloc_forward_refuses_layouts_beyond_its_scratch(sa):
    """The no-allocation forward holds at most 128 MiB of permuted K and V;
    a larger layout is refused before anything touches the device (the
    scratch check precedes the mask check)."""
    h = sa.sparse_attn_create(40, 128, (21, 45, 80), (1, 8, 16), "bf16")  # 1.65 GB of K and V
    L = sa.sparse_attn_layout(h)
    assert 2 * L["ws_offset_k"] > sa.SPARSE_ATTN_NOALLOC_SCRATCH_BYTES
    fake = 1 << 40
    n = 40 * L["tokens"] * 128 * 2
    st = sa._lib.sparse_attn_forward_noalloc(h.ptr, fake, fake + n, fake + 2 * n, fake + 3 * n, None)
    assert st == sa.SPARSE_ATTN_UNSUPPORTED
    assert "no-allocation forward holds at most" in sa.sparse_attn_last_error(h)
    small = sa.sparse_attn_create(12, 128, (8, 30, 40), (1, 8, 16), "bf16")  # 75.5 MB: fits
    Ls = sa.sparse_attn_layout(small)
    assert 2 * Ls["ws_offset_k"] <= sa.SPARSE_ATTN_NOALLOC_SCRATCH_BYTES
    ns = 12 * Ls["tokens"] * 128 * 2
    st = sa._lib.sparse_attn_forward_noalloc(small.ptr, fake, fake + ns, fake + 2 * ns, fake + 3 * ns, None)
    assert st == sa.SPARSE_ATTN_NO_MASK


@pytest.mark.parametrize("waves,cus,iters", [(0, 256, 10), (4, 256, 10), (2, 0, 10), (2, 256, 0),
                                             (2, 256, (1 << 20) + 1)])
def test_mix_probe_rejects_bad_sizes(sa, waves, cus, iters):
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_mix_probe(waves, cus, iters, 1 << 20, 1 << 21, stream=0)
    assert e.value.status == sa.SPARSE_ATTN_INVALID_ARG
    assert "must" in sa.sparse_attn_last_error(None)


def test_mix_probe_pingpong_needs_two_waves_per_simd(sa):
    for waves in (1, 3):
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_mix_probe(waves, 256, 10, 1 << 20, 1 << 21, pingpong=True, stream=0)
        assert e.value.status == sa.SPARSE_ATTN_INVALID_ARG
    assert sa._lib.sparse_attn_mix_probe(2, 2, 256, 10, 1 << 20, 1 << 21, 0) == sa.SPARSE_ATTN_INVALID_ARG


def test_mix_probe_rejects_null_or_misaligned_buffers(sa):
    for cyc, sink in [(None, 1 << 21), (1 << 20, None), ((1 << 20) + 4, 1 << 21), (1 << 20, (1 << 21) + 2)]:
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_mix_probe(2, 256, 10, cyc, sink, stream=0)
        assert e.value.status == sa.SPARSE_ATTN_INVALID_ARG

"""GPU parity of the block-sparse attention forward against the fp64 oracle.

Tolerances: max-abs 1e-5 for fp32, max-abs 2e-2 plus relative RMS 2e-2 for
bf16 inputs.  Small shapes are compared element by element in full; the
720p workloads at full size are compared on sampled query rows (every head:
the first, last, a clipped and the longest-row query tile, plus random
tokens), computed one by one by the oracle."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from workloads import make_workload, ones_bitmap

from gpu_helpers import as_f64, assert_close, dev, host

pytestmark = pytest.mark.gpu


class Case:
    """Inputs of one forward: grid, tile, q/k/v (numpy), mask."""

    def __init__(self, grid, tile, q, k, v, dtype, bitmap=None, groups=None, gph=None, scale=0.0,
                 pairing="auto", vector_alu=False):
        self.grid, self.tile, self.q, self.k, self.v = grid, tile, q, k, v
        self.dtype, self.bitmap, self.groups, self.gph, self.scale = dtype, bitmap, groups, gph, scale
        self.pairing, self.vector_alu = pairing, vector_alu
        self.heads, self.N, self.d = q.shape

    @staticmethod
    def of(wl, bitmap=None):
        if bitmap is not None or wl.mask_kind == "bitmap":
            return Case(wl.grid, wl.tile, wl.q, wl.k, wl.v, wl.dtype,
                        bitmap=wl.bitmap if bitmap is None else bitmap)
        return Case(wl.grid, wl.tile, wl.q, wl.k, wl.v, wl.dtype, groups=wl.groups,
                    gph=wl.groups_per_head)

    def mask(self):
        if self.bitmap is not None:
            return np.ascontiguousarray(self.bitmap != 0, dtype=np.uint8)
        return oracle.mask_from_windows(self.grid, self.tile, self.groups, self.gph)

    def oracle_scale(self):
        return self.scale if self.scale > 0 else 1.0 / np.sqrt(self.d)


def gpu_forward(c, stages=False):
    h = sa.sparse_attn_create(c.heads, c.d, c.grid, c.tile, c.dtype, c.scale, pairing=c.pairing,
                              vector_alu=c.vector_alu)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    if c.bitmap is not None:
        sa.sparse_attn_set_mask(h, mb, bitmap=dev(c.bitmap))
    else:
        sa.sparse_attn_set_mask(h, mb, groups=c.groups, groups_per_head=c.gph)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    o = torch.full_like(q, 0x7FC0 if c.dtype == "bf16" else 0)
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    if stages:
        sa.sparse_attn_permute_inputs(h, q, k, v, ws)
        sa.sparse_attn_attend(h, ws)
        sa.sparse_attn_unpermute_output(h, ws, o)
    else:
        sa.sparse_attn_forward(h, q, k, v, o, ws)
    torch.cuda.synchronize()
    return host(o, c.q), sa.sparse_attn_layout(h)


def full_check(c, what):
    print(f"forward {what} grid={c.grid} tile={c.tile} heads={c.heads} d={c.d} {c.dtype}", flush=True)
    got, layout = gpu_forward(c)
    want = oracle.attention(c.grid, c.tile, c.q, c.k, c.v, c.mask(), scale=c.oracle_scale())
    assert_close(as_f64(got), want, c.dtype, what)
    return got, want, layout


def test_tiny_fp32():
    wl = make_workload("tiny")
    _, _, layout = full_check(Case.of(wl), "tiny")
    assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_F32
    c = Case.of(wl)
    c.vector_alu = True
    _, _, layout = full_check(c, "tiny, vector ALU")
    assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_GENERIC


@pytest.mark.parametrize("pairing", ["auto", "overlap", "all"])
def test_small_bf16(pairing):
    """The Small workload through each work split of the matrix-core path
    (auto runs the row kernel only at this size; overlap splits pairs and
    single tiles; all runs the pair kernel only)."""
    wl = make_workload("small")
    c = Case.of(wl)
    c.pairing = pairing
    got, _, layout = full_check(c, f"small pairing={pairing}")
    assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_BF16
    assert layout["pairing"] == (sa.SPARSE_ATTN_PAIRING_NONE if pairing == "auto" else sa._PAIRINGS[pairing])


def test_small_dense_mask():
    wl = make_workload("small", heads=3)
    full_check(Case.of(wl, bitmap=ones_bitmap(wl)), "small-dense")


def _rand(shape, seed, dtype, scale=1.0):
    from workloads import f32_to_bf16_bits
    x = (np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * scale)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _random_case(grid, tile, d, dtype, heads=3, p=0.4, seed=0, empty_row=True, scale=0.0):
    N = int(np.prod(grid))
    nT = oracle.num_tiles(grid, tile)
    q, k, v = (_rand((heads, N, d), seed + s, dtype) for s in (1, 2, 3))
    rng = np.random.default_rng(seed + 4)
    M = (rng.random((heads, nT, nT)) < p).astype(np.uint8)
    if empty_row:
        M[0, nT // 2, :] = 0
    return Case(grid, tile, q, k, v, dtype, bitmap=M, scale=scale)


@pytest.mark.parametrize("grid,tile,d,dtype", [
    ((3, 20, 36), (1, 8, 16), 128, "bf16"),   # clipped tiles of 128, 64, 32 and 16 tokens
    ((3, 20, 36), (1, 8, 16), 64, "bf16"),    # head_dim 64 on the matrix cores
    ((1, 5, 7), (1, 8, 16), 128, "bf16"),     # one tile, larger than the grid
    ((2, 17, 33), (2, 4, 16), 128, "bf16"),   # clipped along t, y and x
    ((3, 10, 12), (1, 4, 8), 64, "bf16"),     # 32-token tiles in 128-slot blocks
    ((3, 20, 36), (1, 8, 8), 128, "bf16"),    # 64-token tiles, clipped to 32
    ((5, 10, 12), (2, 4, 8), 128, "bf16"),    # 64-token tiles clipped along t, y and x
    ((2, 9, 11), (1, 3, 5), 64, "bf16"),      # 15-token tiles: one partial key block
    ((3, 10, 12), (1, 4, 8), 128, "f32"),
    ((2, 5, 7), (2, 2, 3), 64, "f32"),
])
@pytest.mark.parametrize("pairing", ["auto", "overlap", "all"])  # auto is NONE on these grids
def test_ragged_shapes_with_empty_rows(grid, tile, d, dtype, pairing):
    c = _random_case(grid, tile, d, dtype)
    c.pairing = pairing
    got, want, layout = full_check(c, f"ragged pairing={pairing}")
    # bf16 runs on the matrix cores for every tile volume, in 128-slot blocks.
    B = int(np.prod(tile))
    assert layout["tile_volume"] == B
    if dtype == "bf16":
        assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_BF16 and layout["slot_stride"] == 128
    else:
        assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_F32 and layout["slot_stride"] == B
    nT = oracle.num_tiles(grid, tile)
    # the empty row (head 0, query tile nT // 2) outputs exactly zero
    perm, _ = oracle.perm(grid, tile)
    toks = perm[(nT // 2) * B:(nT // 2 + 1) * B]
    toks = toks[toks >= 0]
    assert np.all(as_f64(got[0, toks]) == 0.0)


@pytest.mark.parametrize("grid,tile,d", [
    ((3, 20, 36), (1, 8, 16), 128),
    ((3, 10, 12), (1, 4, 8), 64),
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_on_the_vector_alu_kernel(grid, tile, d, dtype):
    """bf16 and fp32 inputs on the vector-ALU kernel (on request), tiles of B slots."""
    c = _random_case(grid, tile, d, dtype)
    c.vector_alu = True
    _, _, layout = full_check(c, f"{dtype} vector-ALU")
    assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_GENERIC
    assert layout["slot_stride"] == int(np.prod(tile))


def test_explicit_scale():
    c = _random_case((2, 16, 32), (1, 8, 16), 128, "bf16", scale=0.05, empty_row=False)
    full_check(c, "scale")


def test_all_rows_empty():
    c = _random_case((2, 16, 32), (1, 8, 16), 128, "bf16", p=0.0, empty_row=False)
    got, _ = gpu_forward(c)
    assert np.all(as_f64(got) == 0.0)


# ---------------------------------------------------------------------------
# Probes with closed-form answers


def test_probe_zero_queries_average_real_kept_values():
    # q = 0: every output is the mean of the values of the real keys in kept
    # tiles; counting the empty slots of clipped tiles would shrink it.
    grid, tile, d = (3, 20, 36), (1, 8, 16), 128
    c = _random_case(grid, tile, d, "bf16", p=0.5, empty_row=False)
    c.q = np.zeros_like(c.q)
    got, _ = gpu_forward(c)
    M = c.mask()
    perm, pos = oracle.perm(grid, tile)
    B = int(np.prod(tile))
    tile_of = pos // B
    v = as_f64(c.v)
    want = np.zeros_like(v)
    for h in range(c.heads):
        for i in range(M.shape[1]):
            keys = np.isin(tile_of, np.nonzero(M[h, i])[0])
            toks = tile_of == i
            if keys.any():
                want[h, toks] = v[h, keys].mean(axis=0)
    assert_close(as_f64(got), want, "bf16", "q=0")


def test_probe_constant_values():
    c = _random_case((3, 20, 36), (1, 8, 16), 128, "bf16", p=0.5, empty_row=False)
    c.v = np.full_like(c.v, 0x3FC0)  # 1.5 in bf16
    got, _ = gpu_forward(c)
    assert np.abs(as_f64(got) - 1.5).max() <= 1.5 * 2 ** -7


@pytest.mark.parametrize("dtype,grid,tile,d", [("f32", (4, 8, 8), (1, 4, 4), 64),
                                               ("bf16", (2, 30, 40), (1, 8, 16), 128)])
def test_probe_tile_indicator_values(dtype, grid, tile, d):
    # v[m, tau] = 1 iff token m is in tile tau: column tau of the output is
    # the attention mass on tile tau -- exactly 0 where the mask drops it.
    c = _random_case(grid, tile, d, dtype, p=0.5, empty_row=False)
    nT = oracle.num_tiles(grid, tile)
    B = int(np.prod(tile))
    _, pos = oracle.perm(grid, tile)
    tile_of = pos // B
    one = np.float32(1.0) if dtype == "f32" else np.uint16(0x3F80)
    v = np.zeros_like(c.v)
    v[:, np.arange(c.N), tile_of] = one
    c.v = v
    got = as_f64(gpu_forward(c)[0])
    M = c.mask()
    for h in range(c.heads):
        keep = M[h][tile_of] != 0  # [N, nT]
        assert np.all(got[h][:, :nT][~keep] == 0.0)
        assert np.all(got[h][:, :nT][keep] > 0.0)
        tol = 1e-5 if dtype == "f32" else 2e-2
        assert np.abs(got[h][:, :nT].sum(axis=1) - 1.0).max() <= tol
    want = oracle.attention(grid, tile, c.q, c.k, c.v, M)
    assert_close(got, want, dtype, "tile-indicator")


def test_probe_block_diagonal_mask():
    grid, tile, d = (2, 16, 32), (1, 8, 16), 128
    c = _random_case(grid, tile, d, "bf16", empty_row=False)
    nT = oracle.num_tiles(grid, tile)
    c.bitmap = np.broadcast_to(np.eye(nT, dtype=np.uint8), (c.heads, nT, nT)).copy()
    got, _ = gpu_forward(c)
    # dense attention inside each tile, by library SDPA in float64 on the CPU
    T, H, W = grid
    def tiles(x):
        x = x.reshape(c.heads, T, H // 8, 8, W // 16, 16, d).transpose(0, 1, 2, 4, 3, 5, 6)
        return torch.from_numpy(np.ascontiguousarray(x.reshape(c.heads, nT, 128, d)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tiles(as_f64(c.q)), tiles(as_f64(c.k)), tiles(as_f64(c.v))).numpy()
    assert_close(tiles(as_f64(got)).numpy(), ref, "bf16", "block-diagonal")


# ---------------------------------------------------------------------------
# Determinism and the stage entry points


def test_deterministic_and_stages_equal_forward():
    wl = make_workload("small", heads=4)
    c = Case.of(wl)
    a, _ = gpu_forward(c)
    b, _ = gpu_forward(c)
    s, _ = gpu_forward(c, stages=True)
    assert np.array_equal(a, b) and np.array_equal(a, s)


def test_mask_can_be_replaced_between_forwards():
    wl = make_workload("small", heads=2)
    c = Case.of(wl)
    h = sa.sparse_attn_create(2, 128, wl.grid, wl.tile, "bf16")
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    o = torch.empty_like(q)
    ones = ones_bitmap(wl)
    for bitmap in (c.mask(), ones):
        sa.sparse_attn_set_mask(h, mb, bitmap=dev(bitmap))
        sa.sparse_attn_forward(h, q, k, v, o, ws)
        want = oracle.attention(wl.grid, wl.tile, c.q, c.k, c.v, bitmap)
        assert_close(as_f64(host(o, c.q)), want, "bf16", "replace")


# ---------------------------------------------------------------------------
# The 720p workloads at full size, sampled rows


def _sample_rows(wl, M, per_tile=16, random_rows=32, seed=7):
    B = int(np.prod(wl.tile))
    nT = M.shape[1]
    perm, _ = oracle.perm(wl.grid, wl.tile)
    counts = oracle.tile_counts(wl.grid, wl.tile)
    partial = int(np.nonzero(counts < B)[0][0]) if (counts < B).any() else nT // 2
    rng = np.random.default_rng(seed)
    rows = []
    for h in range(wl.heads):
        longest = int(np.argmax(M[h].sum(axis=1)))
        for t in sorted({0, nT - 1, partial, longest}):
            toks = perm[t * B:t * B + counts[t]]
            rows += (h * wl.config.tokens + rng.choice(toks, size=min(per_tile, len(toks)),
                                                       replace=False)).tolist()
        rows += (h * wl.config.tokens + rng.choice(wl.config.tokens, size=random_rows,
                                                   replace=False)).tolist()
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", ["wan", "hunyuan", "long"])
def test_full_size_workloads_sampled(name):
    wl = make_workload(name)
    print(f"full {name}: heads={wl.heads} density={wl.info['tile_density']:.4f}", flush=True)
    c = Case.of(wl)
    got, layout = gpu_forward(c)
    assert layout["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_BF16
    M = c.mask()
    rows = _sample_rows(wl, M)
    want = oracle.attention_rows(wl.grid, wl.tile, wl.q, wl.k, wl.v, M, rows)
    g = as_f64(got.reshape(-1, wl.head_dim)[rows])
    assert_close(g, want, "bf16", f"{name} ({len(rows)} sampled rows)")
    assert np.all(np.isfinite(as_f64(got[:, ::997])))


def test_forward_on_a_side_stream():
    """Every stage is enqueued on the stream it is given: a forward on a
    separate (default-priority) stream gives the default stream's output."""
    wl = make_workload("small", heads=2)
    c = Case.of(wl)
    want, _ = gpu_forward(c)
    h = sa.sparse_attn_create(c.heads, c.d, c.grid, c.tile, c.dtype)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
        q, k, v = dev(c.q), dev(c.k), dev(c.v)
        o = torch.zeros_like(q)
        ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    side.synchronize()
    torch.cuda.synchronize()
    sa.sparse_attn_set_mask(h, mb, groups=c.groups, groups_per_head=c.gph, stream=side)
    sa.sparse_attn_forward(h, q, k, v, o, ws, stream=side)
    side.synchronize()
    assert np.array_equal(host(o, c.q), want)


def test_convenience_wrapper_matches_the_functional_calls():
    """SparseAttention (one handle, its own mask buffer and workspace) gives
    the functional path's output bit for bit, for a window mask and then for
    a bitmap that needs a larger mask buffer."""
    wl = make_workload("small", heads=2)
    c = Case.of(wl)
    want, _ = gpu_forward(c)
    att = sa.SparseAttention(c.heads, c.d, c.grid, c.tile, c.dtype)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    att.set_mask_windows(c.groups, c.gph, max_nnz=int(c.mask().sum()))
    got = att.forward(q, k, v)
    torch.cuda.synchronize()
    assert np.array_equal(host(got, c.q), want)
    ones = ones_bitmap(wl)
    att.set_mask_bitmap(dev(ones))
    got = att.forward(q, k, v)
    torch.cuda.synchronize()
    want_dense = oracle.attention(wl.grid, wl.tile, c.q, c.k, c.v, ones)
    assert_close(as_f64(host(got, c.q)), want_dense, "bf16", "wrapper dense")
    att.close()
    assert att.h is None
    att.close()  # a second close is a no-op

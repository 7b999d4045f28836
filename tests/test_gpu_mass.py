"""GPU tile mass (sparse_attn_tile_mass) against the oracle's fp64 full
attention, and the search pipeline end to end.

Bound per entry, from the arithmetic: every term exp(s q.k - LSE) is
positive, so A carries a relative error of at most the score error twice
(d 2^-24 s |q| |k|, once in the score and once through the LSE), plus
n 2^-24 for fp32 sums of n positive terms (N keys in the LSE, up to 128 x
128 terms per tile pair)."""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from oracle import search
from workloads import f32_to_bf16_bits, make_workload

from gpu_helpers import as_f64, dev, host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _bound(q, k, want, N):
    d = q.shape[-1]
    qn = max(np.linalg.norm(as_f64(q[h]), axis=-1).max() for h in range(q.shape[0]))
    kn = max(np.linalg.norm(as_f64(k[h]), axis=-1).max() for h in range(k.shape[0]))
    rel = 2 * d * U * qn * kn / math.sqrt(d) + (N + 128 * 128) * U
    return want * rel + 1e-12


def _gpu_mass(q, k, grid, tile):
    heads, N, d = q.shape
    h = sa.sparse_attn_create(heads, d, grid, tile, "bf16")
    nT = sa.sparse_attn_layout(h)["tiles"]
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    mass = torch.full((heads, nT, nT), -1.0, dtype=torch.float32, device="cuda")
    sa.sparse_attn_tile_mass(h, dev(q), dev(k), ws, mass)
    torch.cuda.synchronize()
    return h, mass.cpu().numpy()


@pytest.mark.parametrize("grid,tile,d", [((3, 20, 36), (1, 8, 16), 128), ((2, 17, 33), (2, 4, 16), 64),
                                         ((4, 16, 16), (1, 8, 16), 128),
                                         ((3, 10, 12), (1, 4, 8), 64)])  # 32-token tiles
def test_mass_matches_the_oracle(grid, tile, d):
    heads = 2
    N = int(np.prod(grid))
    rng = np.random.default_rng(3)
    q = f32_to_bf16_bits(rng.standard_normal((heads, N, d)).astype(np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((heads, N, d)).astype(np.float32))
    print(f"tile mass grid={grid} tile={tile} d={d}", flush=True)
    _, got = _gpu_mass(q, k, grid, tile)
    want = oracle.tile_mass(grid, tile, q, k)
    err = np.abs(got - want)
    bound = _bound(q, k, want, N)
    print(f"  max abs {err.max():.3e}, max err/bound {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)


def test_mass_full_size_wan_sampled_tiles():
    wl = make_workload("wan")
    grid, tile, d = wl.grid, wl.tile, wl.head_dim
    N = wl.config.tokens
    print(f"tile mass wan full heads={wl.heads}", flush=True)
    _, got = _gpu_mass(wl.q, wl.k, grid, tile)
    nT = got.shape[1]
    rng = np.random.default_rng(9)
    qt = np.sort(rng.choice(wl.heads * nT, size=12, replace=False))
    want = oracle.tile_mass(grid, tile, wl.q, wl.k, qtiles=qt)
    rows = got.reshape(-1, nT)[qt]
    err = np.abs(rows - want)
    qn = max(np.linalg.norm(as_f64(wl.q[h]), axis=-1).max() for h in range(wl.heads))
    kn = max(np.linalg.norm(as_f64(wl.k[h]), axis=-1).max() for h in range(wl.heads))
    bound = want * (2 * d * U * qn * kn / math.sqrt(d) + (N + 128 * 128) * U) + 1e-12
    print(f"  max abs {err.max():.3e}, max err/bound {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)
    assert np.abs(got.sum(axis=2) - 1).max() < 1e-3


def test_mass_needs_the_matrix_core_path():
    h = sa.sparse_attn_create(2, 64, (4, 8, 8), (1, 4, 4), "f32")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    x = torch.zeros((2, 256, 64), dtype=torch.float32, device="cuda")
    m = torch.empty((2, 16, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_tile_mass(h, x, x, ws, m)
    assert e.value.status == sa.SPARSE_ATTN_UNSUPPORTED


def test_search_pipeline_end_to_end():
    """GPU mass -> host search at tau = 0.9 -> set_mask -> forward: the
    searched windows equal the oracle search's on the GPU mass, the recall
    under the exact mass is tau up to the mass error, and the forward
    matches the oracle's attention under the searched mask."""
    grid, tile, heads, d = (4, 24, 32), (1, 8, 16), 2, 128
    N = int(np.prod(grid))
    rng = np.random.default_rng(12)
    qf, kf, vf = (f32_to_bf16_bits(rng.standard_normal((heads, N, d)).astype(np.float32)) for _ in range(3))
    h, A = _gpu_mass(qf, kf, grid, tile)
    spec = [(0, 0), (1, 2), (3, -1)]
    g_in = np.array([(lo, hi, 0, 0, 0, 0) for lo, hi in spec] * heads, np.int32)
    gph = np.full(heads, len(spec), np.int32)
    groups, rec, cost = sa.sparse_attn_search_windows(h, A, g_in, gph, 0.9)
    counts = oracle.tile_counts(grid, tile)
    want_g, _, _, _ = search.search(grid, tile, counts, A.astype(np.float64), [spec] * heads, 0.9)
    assert np.array_equal(groups, want_g)
    assert np.all(rec >= 0.9) and np.all(cost < 1)
    M = oracle.mask_from_windows(grid, tile, groups, gph)
    exact = oracle.tile_mass(grid, tile, qf, kf)
    exact_rec = (counts[None, :, None] * exact * M).sum(axis=(1, 2)) / counts.sum()
    assert np.all(exact_rec >= 0.9 - 1e-3), exact_rec
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, groups=groups, groups_per_head=gph)
    q, k, v = dev(qf), dev(kf), dev(vf)
    o = torch.empty_like(q)
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_forward(h, q, k, v, o, ws)
    torch.cuda.synchronize()
    rows = np.random.default_rng(4).choice(heads * N, 256, replace=False)
    want = oracle.attention_rows(grid, tile, qf, kf, vf, M, rows)
    got = as_f64(host(o, qf)).reshape(-1, d)[rows]
    assert np.abs(got - want).max() <= 2e-2
    print(f"  searched density {cost.mean():.3f}, recall {rec.mean():.4f}", flush=True)

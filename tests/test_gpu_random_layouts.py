"""Seeded random layouts through the fused forward with LSE, against the
oracle, each compared in full.

Every case draws a grid ragged in all three axes (T 1-4, H 1-40, W 1-48), a
tile shape of any volume up to 128 (so tiles larger than the grid and
clipped edge tiles appear), head dim 64 or 128, the element type (bf16 on
the matrix cores, bf16 on the vector ALUs, fp32), the token order (tile
boxes or Hilbert runs), the work split (AUTO, OVERLAP, ALL, NONE) and a mask
density from empty to full, with one query tile of the first head emptied.
O must be within the dtype's tolerance of the oracle and exactly 0 on rows
that keep nothing; the LSE within the per-row bound derived from the
kernels' arithmetic (gpu_helpers.lse_bound) and -inf exactly on empty rows
(Compact Attention page, Fig. 3 caption: precomputed tile masks run in
block-sparse kernels; SCOPE review page, abstract: exact attention over the
kept keys)."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from workloads import f32_to_bf16_bits

from gpu_helpers import as_f64, assert_close, assert_lse_close, dev, host, lse_bound

pytestmark = pytest.mark.gpu

CASES = 200


def _draw(i):
    rng = np.random.default_rng(7000 + i)
    grid = (int(rng.integers(1, 5)), int(rng.integers(1, 41)), int(rng.integers(1, 49)))
    while True:
        tile = (int(rng.integers(1, 3)), int(rng.integers(1, 9)), int(rng.integers(1, 17)))
        if np.prod(tile) <= 128:
            break
    return dict(grid=grid, tile=tile, d=int(rng.choice([64, 128])),
                kind=str(rng.choice(["bf16", "bf16", "bf16", "bf16-vector", "f32", "f32-vector"])),
                order=str(rng.choice(["tiles", "hilbert"])),
                pairing=str(rng.choice(["auto", "overlap", "all", "none"])),
                density=float(rng.choice([0.0, 0.15, 0.4, 0.7, 1.0], p=[0.05, 0.3, 0.3, 0.2, 0.15])),
                heads=int(rng.integers(1, 4)), seed=7000 + i)


@pytest.mark.parametrize("i", range(CASES))
def test_random_layout(i):
    c = _draw(i)
    grid, tile, d, heads = c["grid"], c["tile"], c["d"], c["heads"]
    dtype = c["kind"].split("-")[0]
    print(f"random layout {i}: {c}", flush=True)
    N = int(np.prod(grid))
    B = int(np.prod(tile))
    # The oracle's view of the layout: the grid itself (tile boxes), or the
    # tokens in Hilbert rank order as a 1 x 1 x N grid of 1 x 1 x B tiles.
    if c["order"] == "hilbert":
        seq = oracle.hilbert_order(grid)
        g1, t1 = (1, 1, N), (1, 1, B)
    else:
        seq = np.arange(N)
        g1, t1 = grid, tile
    nT = oracle.num_tiles(g1, t1)
    rng = np.random.default_rng(c["seed"])
    x = [rng.standard_normal((heads, N, d), dtype=np.float32) for _ in range(3)]
    q, k, v = (a if dtype == "f32" else f32_to_bf16_bits(a) for a in x)
    M = (rng.random((heads, nT, nT)) < c["density"]).astype(np.uint8)
    M[0, nT // 2] = 0

    h = sa.sparse_attn_create(heads, d, grid, tile, dtype, order=c["order"], pairing=c["pairing"],
                              vector_alu=c["kind"].endswith("-vector"))
    keep = []
    if c["order"] == "hilbert":
        ob = torch.empty(sa.sparse_attn_order_bytes(h), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_set_order(h, ob)
        keep.append(ob)
    L = sa.sparse_attn_layout(h)
    assert L["tiles"] == nT and L["tile_volume"] == B
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, bitmap=dev(M))
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.full_like(qd, 0x7FC0 if dtype == "bf16" else 0)
    lse = torch.full((heads, N), 12345.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_forward_lse(h, qd, kd, vd, o, lse, ws)
    torch.cuda.synchronize()
    nnz, overflow = sa.sparse_attn_mask_info(h)
    assert not overflow and nnz == int(M.sum())
    got, got_lse = as_f64(host(o, q)), lse.cpu().numpy().astype(np.float64)

    want_s, lse_s = oracle.attention(g1, t1, q[:, seq], k[:, seq], v[:, seq], M, lse=True)
    want = np.empty_like(want_s)
    want[:, seq] = want_s
    want_lse = np.empty_like(lse_s)
    want_lse[:, seq] = lse_s
    assert_close(got, want, dtype, f"case {i} o")
    empty = np.isneginf(want_lse)
    assert np.all(got[empty] == 0.0)
    _, pos = oracle.perm(g1, t1)
    kept_s = (M.astype(np.int64) @ oracle.tile_counts(g1, t1))[:, pos // B]
    kept = np.empty_like(kept_s)
    kept[:, seq] = kept_s
    kmax = np.array([np.linalg.norm(as_f64(k[hh]), axis=-1).max() for hh in range(heads)])
    bound = lse_bound(as_f64(q).reshape(-1, d), np.repeat(kmax, N), kept.reshape(-1), d,
                      1.0 / np.sqrt(d), dtype, want_lse.reshape(-1))
    assert_lse_close(got_lse.reshape(-1), want_lse.reshape(-1), bound, f"case {i}")

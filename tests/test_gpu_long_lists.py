"""GPU parity with key lists longer than the kernels stage in LDS at once.

Both attention kernels keep at most 2,048 list entries in LDS and reload
the rest as their cursor advances (the pair kernel into the free half of a
ring, the row kernel after a barrier).  No 720p workload has lists that
long (at most 1,260 tiles), so this case builds them: 2,600 tiles per head
(grid 26 x 80 x 160, tiles 1 x 8 x 16).  Head 0: the query tiles of frames
0-1 keep every key tile, so their y-neighbour pairs share lists of 2,600
entries (pair kernel); in frame 5 the even tile rows keep every key tile
and the odd rows only themselves, so those pairs fail the sharing test and
the dense rows run on the row kernel.  Head 1: frames 10-11 keep each key
tile with probability 0.85 (about 2,200 entries per row).  Every other
query tile keeps itself and one scattered tile.  Sampled query rows of
those frames and elsewhere are compared with the oracle."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle

from gpu_helpers import as_f64, assert_close, assert_lse_close, dev, host, lse_bound

pytestmark = pytest.mark.gpu

GRID, TILE, D, HEADS = (26, 80, 160), (1, 8, 16), 128, 2
NY, NX = 10, 10


def _bf16_bits(rng, n):
    """Random bf16 bit patterns of magnitude 0.5-2 with random signs."""
    r = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    return (r & np.uint16(0x80FF)) | np.uint16(0x3F00)


def _bitmap(nT, rng):
    i = np.arange(nT)
    a, b = i // (NY * NX), (i // NX) % NY
    M = np.zeros((HEADS, nT, nT), dtype=np.uint8)
    M[:, i, i] = 1
    M[:, i, (i * 7919 + 13) % nT] = 1
    M[0, a < 2, :] = 1
    M[0, (a == 5) & (b % 2 == 0), :] = 1
    rows = np.nonzero((a == 10) | (a == 11))[0]
    M[1, rows, :] |= (rng.random((len(rows), nT)) < 0.85).astype(np.uint8)
    return M


def test_lists_longer_than_the_lds_stage():
    h = sa.sparse_attn_create(HEADS, D, GRID, TILE, "bf16")
    L = sa.sparse_attn_layout(h)
    nT, N = L["tiles"], L["tokens"]
    assert nT == 2600 and L["pair_axis"] == 1
    rng = np.random.default_rng(31)
    q, k, v = (_bf16_bits(rng, HEADS * N * D).reshape(HEADS, N, D) for _ in range(3))
    M = _bitmap(nT, rng)
    lens = M.sum(axis=2)
    assert lens.max() == nT and (lens[1] > 2048).sum() >= 150
    print(f"long lists: {nT} tiles, longest rows {lens.max()}, {int((lens > 2048).sum())} rows over 2048",
          flush=True)
    nnz = int(M.sum())
    mb = torch.empty(sa.sparse_attn_mask_bytes(h, nnz), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, bitmap=dev(M), max_nnz=nnz)

    # Which kernel serves the long rows: pair flags of the pairs involved.
    P = HEADS * L["pairs"]  # pair rows of all heads
    i32 = dict(dtype=torch.int32, device="cuda")
    rp, cols, order, flag = (torch.empty(P + 1, **i32), torch.empty(nnz, **i32),
                             torch.empty(P, **i32), torch.empty(P, **i32))
    sa.sparse_attn_read_pair_lists(h, rp, cols, order, flag)
    flag = flag.cpu().numpy().reshape(HEADS, -1)
    plen = np.diff(rp.cpu().numpy()).reshape(HEADS, -1)
    per_frame = (NY // 2) * NX
    assert flag[0, :2 * per_frame].all() and (plen[0, :2 * per_frame] == nT).all()
    assert not flag[0, 5 * per_frame:6 * per_frame].any()
    assert flag[1, 10 * per_frame:12 * per_frame].all() and (plen[1, 10 * per_frame:12 * per_frame] > 2048).all()

    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.full_like(qd, 0x7FC0)
    lse = torch.full((HEADS, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_forward_lse(h, qd, kd, vd, o, lse, ws)
    torch.cuda.synchronize()

    frame = GRID[1] * GRID[2]
    pick = lambda hh, f, n: hh * N + f * frame + rng.choice(frame, n, replace=False)
    rows = np.unique(np.concatenate([
        pick(0, 0, 24), pick(0, 1, 24), pick(0, 5, 40), pick(1, 10, 24), pick(1, 11, 24),
        rng.choice(HEADS * N, 24, replace=False)])).astype(np.int64)
    print(f"  oracle on {len(rows)} sampled rows", flush=True)
    want, want_lse = oracle.attention_rows(GRID, TILE, q, k, v, M, rows, lse=True)
    got = as_f64(host(o, q).reshape(-1, D)[rows])
    assert_close(got, want, "bf16", f"long lists ({len(rows)} sampled rows)")
    # Every tile is full (128 tokens); features are below 2 in magnitude.
    hh, n = rows // N, rows % N
    tile_of = (n // frame) * NY * NX + ((n % frame) // GRID[2] // 8) * NX + (n % GRID[2]) // 16
    kept = M[hh, tile_of].sum(axis=1) * 128
    bound = lse_bound(as_f64(q.reshape(-1, D)[rows]), 2.0 * np.sqrt(D), kept, D, 1.0 / np.sqrt(D), "bf16",
                      want_lse)
    assert_lse_close(lse.cpu().numpy().reshape(-1)[rows].astype(np.float64), want_lse, bound, "long lists")
    sa.sparse_attn_destroy(h)

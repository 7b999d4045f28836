"""GPU parity at the largest layout the plan accepts for one head.

heads * tiles^2 must stay below 2^31, so one head takes at most 46,340
tiles: grid 331 x 80 x 224 with 1 x 8 x 16 tiles (5,931,520 tokens, every
tile full).  K and the transposed V of the head then span 1.52e9 bytes,
the largest 32-bit stage offsets and buffer ranges the attention kernels
use, and the tile bitmap is 2.15e9 bytes.  The mask keeps, per query tile
(a, b, e), the tile itself, the top tile (a, 0, e) of its column and the
far tile (330 - a, 9, 13 - e) (query tile 0 keeps the last tile), so two
tiles neighbouring along y share two of their keys and the pair kernel
takes them; tiles of frames 300 and up also keep three scattered tiles,
so their pairs share too little and go to the row kernel.
Inputs are random bf16 values of magnitude 0.5-2 with random signs (drawn
as bit patterns, which is fast at this size).  Sampled query rows are
compared with the oracle, outputs and log-sum-exp."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle

from gpu_helpers import as_f64, assert_close, assert_lse_close, dev, host, lse_bound

pytestmark = pytest.mark.gpu

GRID, TILE, D = (331, 80, 224), (1, 8, 16), 128
NT, NY, NX = 331, 10, 14


def _bf16_bits(rng, n):
    """Random bf16 bit patterns: sign from bit 15, exponent 126 or 127 and
    7 random mantissa bits, i.e. magnitudes in [0.5, 2)."""
    r = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    return (r & np.uint16(0x80FF)) | np.uint16(0x3F00)


def _bitmap(nT):
    i = np.arange(nT, dtype=np.int64)
    a, e = i // (NY * NX), i % NX
    M = np.zeros((1, nT, nT), dtype=np.uint8)
    M[0, i, i] = 1
    M[0, i, a * NY * NX + e] = 1                                    # top tile of the column
    M[0, i, ((NT - 1 - a) * NY + NY - 1) * NX + (NX - 1 - e)] = 1   # far tile
    late = i[a >= 300]
    for mul in (7919, 104729, 15485863):
        M[0, late, (late * mul) % nT] = 1
    return M


def test_largest_layout_sampled():
    h = sa.sparse_attn_create(1, D, GRID, TILE, "bf16")
    L = sa.sparse_attn_layout(h)
    nT, N = L["tiles"], L["tokens"]
    assert nT == 46340 and N == 5931520 and L["slots"] == N
    print(f"largest layout: {nT} tiles, {N} tokens; drawing inputs", flush=True)
    rng = np.random.default_rng(2026)
    q, k, v = (_bf16_bits(rng, N * D).reshape(1, N, D) for _ in range(3))
    M = _bitmap(nT)
    nnz = int(M.sum())
    print(f"  bitmap {M.nbytes / 1e9:.2f} GB, {nnz} kept tile pairs; set_mask + forward", flush=True)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h, nnz), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, bitmap=dev(M), max_nnz=nnz)
    got_nnz, overflow = sa.sparse_attn_mask_info(h)
    assert got_nnz == nnz and not overflow
    # Query tiles pair along y (5 pairs per column): pairs of frames below
    # 300 run on the pair kernel, the rest on the row kernel.
    assert L["pair_axis"] == 1 and L["pair_grid"] == [NT, NY // 2, NX]
    P = L["pairs"]  # pair rows of the one head
    i32 = dict(dtype=torch.int32, device="cuda")
    rp, cols, order, flag = (torch.empty(P + 1, **i32), torch.empty(nnz, **i32),
                             torch.empty(P, **i32), torch.empty(P, **i32))
    sa.sparse_attn_read_pair_lists(h, rp, cols, order, flag)
    frame_of_pair = np.arange(P) // ((NY // 2) * NX)
    assert np.array_equal(flag.cpu().numpy() != 0, frame_of_pair < 300)
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.full_like(qd, 0x7FC0)
    lse = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_forward_lse(h, qd, kd, vd, o, lse, ws)
    torch.cuda.synchronize()

    frame = GRID[1] * GRID[2]
    rows = np.unique(np.concatenate([
        np.arange(64), np.arange(N - 64, N),                     # first and last tiles
        299 * frame + rng.choice(frame, 48, replace=False),      # pair kernel, far keys
        300 * frame + rng.choice(frame, 48, replace=False),      # row kernel
        330 * frame + rng.choice(frame, 48, replace=False),
        rng.choice(N, 96, replace=False)])).astype(np.int64)
    print(f"  oracle on {len(rows)} sampled rows", flush=True)
    want, want_lse = oracle.attention_rows(GRID, TILE, q, k, v, M, rows, lse=True)
    got = as_f64(host(o, q).reshape(-1, D)[rows])
    assert_close(got, want, "bf16", f"largest layout ({len(rows)} sampled rows)")
    got_lse = lse.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    qf = as_f64(q.reshape(-1, D)[rows])
    kmax = 2.0 * np.sqrt(D)  # every feature of every key is below 2 in magnitude
    tiles_of_row = M[0].sum(axis=1)[(rows // frame) * NY * NX + ((rows % frame) // GRID[2] // 8) * NX
                                    + (rows % GRID[2]) // 16]
    bound = lse_bound(qf, kmax, tiles_of_row * 128, D, 1.0 / np.sqrt(D), "bf16", want_lse)
    assert_lse_close(got_lse, want_lse, bound, "largest layout")
    sa.sparse_attn_destroy(h)

"""Closed-form probes over every query row of all five workloads, at full
size, through the fused forward with LSE (the bench's launch configuration).

With Q = 0 every kept score is exactly 0, so every kept key weighs exactly 1
(exp2(0) = 1, exact in bf16 and fp32) and, for a query in tile i of head h:
  - exp(LSE) = sum_j M_h[i, j] c_j, an integer below 2^24, summed exactly;
  - with the probe values V[m, f] = 1 if tile(m) mod d == f else 0,
    O[f] = X_h[i, f] / count, X_h[i, f] = sum_{j kept, j mod d = f} c_j,
    an exact integer ratio; the kernels sum integers (exact in fp32) and
    divide once, so O carries only the final roundings.
A dropped or duplicated kept tile j changes the count by c_j >= 1 (LSE by
>= ln(1 + 1/count), far above its rounding) and one feature of O by about
c_j / X (a large fraction of it).  This is the sharp check the sampled
2e-2 gate cannot give on long rows (Compact Attention page, Fig. 3 caption:
masked tiles run in block-sparse kernels, so every kept tile must be used
exactly once; SCOPE review page, abstract: exact attention over the kept
keys).  Expected values come from the oracle's mask, tile counts and
permutation; the comparison runs on the device to spare copying O back."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
import oracle
from workloads import make_workload

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _expected(wl):
    """count [heads, nT] and X [heads, nT, d] from the oracle's mask."""
    M = oracle.mask_of(wl).astype(np.float64)
    c = oracle.tile_counts(wl.grid, wl.tile).astype(np.float64)
    nT, d = c.shape[0], wl.head_dim
    C = np.zeros((nT, d))
    C[np.arange(nT), np.arange(nT) % d] = c
    count = M @ c                       # [heads, nT]
    X = M @ C                           # [heads, nT, d]
    return count, X


@pytest.mark.parametrize("name", ["tiny", "small", "wan", "hunyuan", "long"])
def test_zero_query_probe_every_row(name):
    wl = make_workload(name, masks_only=True)
    heads, d, N = wl.heads, wl.head_dim, wl.config.tokens
    print(f"probe {name}: heads={heads} tokens={N} d={d} {wl.dtype}", flush=True)
    count, X = _expected(wl)
    assert count.max() < 2 ** 24
    _, pos = oracle.perm(wl.grid, wl.tile)
    B = int(np.prod(wl.tile))
    tile_of = torch.from_numpy((pos // B).astype(np.int64)).cuda()          # [N]
    tdtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    onehot = (tile_of[:, None] % d == torch.arange(d, device="cuda")[None, :]).to(tdtype)
    v = onehot[None].expand(heads, N, d).contiguous()
    q = torch.zeros_like(v)
    rng = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn((heads, N, d), generator=rng, device="cuda").to(tdtype)
    o = torch.full_like(v, float("nan"))
    lse = torch.full((heads, N), float("nan"), dtype=torch.float32, device="cuda")

    h = sa.sparse_attn_create(heads, d, wl.grid, wl.tile, wl.dtype)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    if wl.mask_kind == "bitmap":
        sa.sparse_attn_set_mask(h, mb, bitmap=torch.from_numpy(wl.bitmap).cuda())
    else:
        sa.sparse_attn_set_mask(h, mb, groups=wl.groups, groups_per_head=wl.groups_per_head)
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    as_bits = (lambda t: t.view(torch.int16)) if wl.dtype == "bf16" else (lambda t: t)
    sa.sparse_attn_forward_lse(h, as_bits(q), as_bits(k), as_bits(v), as_bits(o), lse, ws)
    torch.cuda.synchronize()
    nnz, overflow = sa.sparse_attn_mask_info(h)
    assert not overflow and nnz == int(oracle.mask_of(wl).sum())

    cnt = torch.from_numpy(count).cuda()[:, tile_of]                          # [heads, N] f64
    # LSE = ln(count): the row sum is exact, so only log2, the final scaling
    # and their roundings remain (a few ulp of max(1, |LSE|)); -inf where
    # the row keeps nothing.
    empty = cnt == 0
    assert torch.equal(torch.isneginf(lse), empty)
    want_lse = torch.log(cnt.clamp(min=1))
    lse_err = (lse.double() - want_lse).abs()[~empty]
    lse_tol = 8 * U * torch.clamp(want_lse.abs(), min=1.0)[~empty]
    worst = float((lse_err / lse_tol).max()) if lse_err.numel() else 0.0
    print(f"  LSE: max |err| {float(lse_err.max()):.3e}, max err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0
    # exp(LSE) identifies the count: its relative error stays below half the
    # gap to the next integer (1 / count) and below 1e-5.
    rel = (torch.exp(lse.double()) / cnt.clamp(min=1) - 1).abs()[~empty]
    gap = (0.5 / cnt.clamp(min=1))[~empty]
    print(f"  exp(LSE) vs count: max relative error {float(rel.max()):.3e}", flush=True)
    assert float(rel.max()) <= 1e-5 and bool((rel < gap).all())

    # O = X / count per feature, per row: fp32 division (correctly rounded
    # reciprocal and product: two roundings) then, on the bf16 path, one
    # rounding to an 8-bit significand (2^-8 relative).
    for hh in range(heads):
        Xh = torch.from_numpy(X[hh]).cuda()[tile_of]                           # [N, d]
        want = Xh / cnt[hh].clamp(min=1)[:, None]
        got = o[hh].double()
        tol = (2.0 ** -8 if wl.dtype == "bf16" else 0.0) + 3 * U
        err = (got - want).abs()
        bad = err > tol * want.abs() + 1e-30
        if bad.any():
            n = int(bad.nonzero()[0, 0])
            raise AssertionError(f"head {hh} token {n}: got {got[n].tolist()[:8]}, want {want[n].tolist()[:8]}")
    print(f"  O: every row within (2^-8 + 3 u) relative", flush=True)

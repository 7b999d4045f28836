"""The host-side list validator on masks the GPU compiler built: every
workload's row and pair lists pass, in both token orders, and a corrupted
copy of a pair list is reported."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
from block_sparse_attention_major_amd import validate
from workloads import make_workload

from gpu_helpers import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "small", "wan", "hunyuan", "long"])
def test_compiled_workload_masks_validate(name):
    wl = make_workload(name, masks_only=True)
    h = sa.sparse_attn_create(wl.heads, wl.head_dim, wl.grid, wl.tile, wl.dtype)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h, wl.info["nnz"]), dtype=torch.uint8, device="cuda")
    if wl.mask_kind == "bitmap":
        sa.sparse_attn_set_mask(h, mb, bitmap=dev(wl.bitmap), max_nnz=wl.info["nnz"])
    else:
        sa.sparse_attn_set_mask(h, mb, groups=wl.groups, groups_per_head=wl.groups_per_head,
                                max_nnz=wl.info["nnz"])
    s = validate.check_compiled_mask(h)
    print(f"validate {name}: {s}", flush=True)
    assert s["nnz"] == wl.info["nnz"]


def test_hilbert_lists_validate_and_a_corrupted_pair_list_is_reported():
    grid, tile, heads = (3, 17, 33), (1, 8, 16), 2
    # OVERLAP (a layout this small would run AUTO as NONE: no pair lists)
    h = sa.sparse_attn_create(heads, 128, grid, tile, "bf16", order="hilbert", pairing="overlap")
    ob = torch.empty(sa.sparse_attn_order_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_order(h, ob)
    L = sa.sparse_attn_layout(h)
    nT = L["tiles"]
    i = np.arange(nT)
    band = (np.abs(i[:, None] - i[None, :]) <= 1).astype(np.uint8)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, bitmap=dev(np.stack([band] * heads)))
    s = validate.check_compiled_mask(h)
    assert s["pairs_served"] > 0
    # Read the lists back, flip one keep bit of a served pair's entry.
    R, P = heads * nT, heads * L["pairs"]
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")
    rp, cl, od = i32(R + 1), i32(s["nnz"]), i32(R)
    sa.sparse_attn_read_index_lists(h, rp, cl, od)
    prp, pcl, pod, pfl = i32(P + 1), i32(s["nnz"]), i32(P), i32(P)
    sa.sparse_attn_read_pair_lists(h, prp, pcl, pod, pfl)
    torch.cuda.synchronize()
    n = lambda t: t.cpu().numpy().astype(np.int64)
    rows = validate.check_row_lists(n(rp), n(cl), n(od), nT, s["nnz"])
    counts = validate._tile_counts(h, L)
    pcl_h = n(pcl)[:int(n(prp)[-1])].copy()
    validate.check_pair_lists(rows, n(prp), pcl_h, n(pod), n(pfl), L, counts, heads)
    pcl_h[0] ^= 1 << 24
    with pytest.raises(ValueError):
        validate.check_pair_lists(rows, n(prp), pcl_h, n(pod), n(pfl), L, counts, heads)

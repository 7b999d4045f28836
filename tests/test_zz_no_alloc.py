"""sparse_attn_forward_noalloc (no caller workspace: the permuted K and V go
to the library's fixed per-device scratch array) against sparse_attn_forward
on the same inputs, bit for bit: the same kernels run on the same data,
only the buffer holding the permuted K and V differs.  Two calls in a row,
the second on a smaller input, then the first shape again, on the
bf16 matrix-core path (tile volume 128), the fp32 matrix-core path and
the Hilbert order."""

import numpy as np
import pytest
import torch

import block_sparse_attention_major_amd as sa
from workloads import make_workload

from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _both(h, q, k, v):
    """(forward with a workspace, forward without) on one handle."""
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    o_ws = torch.full_like(q, 0x7FC0 if q.dtype == torch.int16 else 0)
    o_na = torch.full_like(q, 0x7FC0 if q.dtype == torch.int16 else 0)
    sa.sparse_attn_forward(h, q, k, v, o_ws, ws)
    sa.sparse_attn_forward_noalloc(h, q, k, v, o_na)
    torch.cuda.synchronize()
    return o_ws, o_na


def _handle(wl, order="tiles"):
    h = sa.sparse_attn_create(wl.heads, wl.head_dim, wl.grid, wl.tile, wl.dtype, order=order)
    keep = []
    if order == "hilbert":
        ob = torch.empty(sa.sparse_attn_order_bytes(h), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_set_order(h, ob)
        keep.append(ob)
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    if wl.mask_kind == "bitmap" or order == "hilbert":
        nT = sa.sparse_attn_layout(h)["tiles"]
        rng = np.random.default_rng(9)
        bm = (rng.random((wl.heads, nT, nT)) < 0.4).astype(np.uint8)
        sa.sparse_attn_set_mask(h, mb, bitmap=dev(bm))
    else:
        sa.sparse_attn_set_mask(h, mb, groups=wl.groups, groups_per_head=wl.groups_per_head)
    keep.append(mb)
    return h, keep


@pytest.mark.parametrize("order", ["tiles", "hilbert"])
def test_noalloc_equals_forward_then_smaller_then_again(order):
    big = make_workload("small")             # 12 heads, 75.5 MB of permuted K and V
    little = make_workload("small", heads=3)
    hb, kb = _handle(big, order)
    hl, kl = _handle(little, order)
    print(f"noalloc {order}: {big.heads} heads, then {little.heads}, then {big.heads}", flush=True)
    qb, kkb, vb = dev(big.q), dev(big.k), dev(big.v)
    ql, kkl, vl = dev(little.q), dev(little.k), dev(little.v)
    a_ws, a_na = _both(hb, qb, kkb, vb)
    assert torch.equal(a_ws, a_na)
    b_ws, b_na = _both(hl, ql, kkl, vl)
    assert torch.equal(b_ws, b_na)
    c_ws, c_na = _both(hb, qb, kkb, vb)  # the scratch now holds the smaller call's data
    assert torch.equal(c_ws, c_na) and torch.equal(c_na, a_na)


def test_noalloc_fp32_path():
    wl = make_workload("tiny")
    h, keep = _handle(wl)
    assert sa.sparse_attn_layout(h)["kernel"] == sa.SPARSE_ATTN_KERNEL_MFMA_F32
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    o_ws, o_na = _both(h, q, k, v)
    assert torch.equal(o_ws, o_na)


def test_noalloc_refuses_a_layout_beyond_the_scratch():
    h = sa.sparse_attn_create(40, 128, (21, 45, 80), (1, 8, 16), "bf16")
    N = 21 * 45 * 80
    x = torch.zeros((40, N, 128), dtype=torch.int16, device="cuda")
    o = torch.full_like(x, 0x7FC0)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_forward_noalloc(h, x, x, x, o)
    assert e.value.status == sa.SPARSE_ATTN_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((o == 0x7FC0).all())

"""Benchmark: block-sparse attention forward on one MI355X.

One step is one pass of the whole hot path over the Wan2.1-shaped 720p
workload (40 heads, head_dim 128, bf16, grid 21x45x80 = 75,600 tokens, tile
1x8x16, local / axial / near-dense dual-window masks at ~26% tile density):
mask compile -> permute K/V to tile-major -> block-sparse attention, which
reads Q and writes O in raster order itself.  Inputs are synthetic and
resident in HBM before timing.

Printed: one JSON line.  `value` is the effective throughput of the whole
step, F_alg / step time, where F_alg = 4 d sum over kept tile pairs of
c_i c_j (real tokens only).  `roofline` reports the attention kernel alone
against the bf16 dense matrix peak; `attention.dense_speedup` is the same
kernel's time with an all-ones mask divided by its time with the real mask.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload (rank 0, N = 1 only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan]
                       [--no-cpu-baseline] [--copy-calibration]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 FLOP/clk x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "block-sparse attn fwd effective TFLOP/s + % MFMA peak; speedup vs dense mask"
WORKLOAD_NAMES = {
    "wan": "wan2.1-shaped 720p: 40 heads x 75,600 tokens, d=128, tile 1x8x16, dual-window masks",
    "hunyuan": "hunyuanvideo-shaped 720p: 24 heads x 118,800 tokens, d=128, tile 1x8x16, top-k tile masks",
    "long": "long-video stress: 40 heads x 151,200 tokens, d=128, tile 1x8x16, +-4 frame axial masks",
    "small": "small video: 12 heads x 9,600 tokens, d=128, tile 1x8x16, dual-window masks",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_{}_traffic.json")  # per workload
# The attention stage's two kernels, and the files that decide their work
# split and layout; counter results taken on other versions of these are
# not reported.
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_attention_major_amd", "csrc", f)
                  for f in ("attn_mfma.hip", "attn_rows.hip", "mfma_util.h", "mask.hip", "common.h")]
ATTN_KERNELS = "attn_mfma_kernel<128> (query-tile pairs) + attn_rows_kernel<128> (single tiles)"


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_per_launch(workload):
    """HBM bytes per attention launch from committed counter runs, or None if
    they were taken on another version of the kernel or workload."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, M, budget_s=15.0):
    """Time the fp64 oracle on sampled query rows of the workload."""
    import oracle

    threads = oracle.default_threads()
    N, d = wl.config.tokens, wl.head_dim
    counts = oracle.tile_counts(wl.grid, wl.tile).astype(np.float64)
    _, pos = oracle.perm(wl.grid, wl.tile)
    tile_of = pos // int(np.prod(wl.tile))
    keys_per_row = np.stack([M[h].astype(np.float64) @ counts for h in range(wl.heads)])  # [heads, nT]
    rng = np.random.default_rng(12345)

    def rows_flops(n):
        rows = rng.choice(wl.heads * N, size=n, replace=False)
        f = 4.0 * d * keys_per_row[rows // N, tile_of[rows % N]].sum()
        return np.sort(rows).astype(np.int64), f

    rows, f = rows_flops(max(64, threads * 8))  # calibration
    t0 = time.perf_counter()
    oracle.attention_rows(wl.grid, wl.tile, wl.q, wl.k, wl.v, M, rows, threads=threads)
    rate = f / (time.perf_counter() - t0)
    n = int(min(wl.heads * N, max(64, budget_s * rate / (f / len(rows)))))
    rows, f = rows_flops(n)
    t0 = time.perf_counter()
    oracle.attention_rows(wl.grid, wl.tile, wl.q, wl.k, wl.v, M, rows, threads=threads)
    dt = time.perf_counter() - t0
    F_full = wl.info["flops_alg"]
    return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly over all heads and tokens of the workload "
                      f"({f / 1e12:.3f} TFLOP algorithmic, {dt:.1f} s wall, fp64, OpenMP)",
            "seconds": dt,
            "full_workload_s_extrapolated": F_full / (f / dt),
            "full_workload_note": "the whole workload's oracle time, extrapolated from the sample's rate "
                                  "by algorithmic FLOPs (not measured)"}


def input_fingerprint(wl):
    """Seed and short hashes of the workload's mask description and inputs,
    so a bench record names exactly what it measured."""
    def h(*arrays):
        d = hashlib.blake2b(digest_size=8)
        for a in arrays:
            d.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1))
        return d.hexdigest()
    mask = h(wl.bitmap) if wl.mask_kind == "bitmap" else h(wl.groups, wl.groups_per_head)
    return {"seed": wl.config.seed, "mask_hash": mask, "qkv_hash": h(wl.q, wl.k, wl.v),
            "hash": "blake2b-64 of the raw bytes"}


def topk_order_comparison(sa, wl, q, k, v, density, stream):
    """Top-k masks at the given tile density, chosen by the GPU selection on
    each token order (tile boxes, Hilbert runs), then the fused forward's
    attention stage timed on each.  F_alg = 4 d sum_h c^T M_h c over the
    selected mask, c the tiles' real token counts."""
    import torch
    E = lambda: torch.cuda.Event(enable_timing=True)
    out = {}
    for order in ("tiles", "hilbert"):
        h = sa.sparse_attn_create(wl.heads, wl.head_dim, wl.grid, wl.tile, wl.dtype, order=order)
        L = sa.sparse_attn_layout(h)
        ob = torch.empty(max(16, sa.sparse_attn_order_bytes(h)), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_set_order(h, ob)
        nT, B = L["tiles"], L["tile_volume"]
        kk = max(1, round(density * nT))
        ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_permute_inputs(h, q, k, v, ws)
        bm = torch.empty((wl.heads, nT, nT), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_select_topk(h, [kk] * wl.heads, ws, bm)
        mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_set_mask(h, mb, bitmap=bm)
        o = torch.empty_like(q)
        sa.sparse_attn_permute_kv(h, k, v, ws)
        for _ in range(2):
            sa.sparse_attn_attend_raster(h, q, o, ws)
        ev = []
        for _ in range(5):
            a, b = E(), E()
            a.record(stream)
            sa.sparse_attn_attend_raster(h, q, o, ws)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        if order == "tiles":
            c = np.array([min(wl.tile[0], wl.grid[0] - a * wl.tile[0]) * min(wl.tile[1], wl.grid[1] - b * wl.tile[1])
                          * min(wl.tile[2], wl.grid[2] - e * wl.tile[2])
                          for a in range(L["tile_grid"][0]) for b in range(L["tile_grid"][1])
                          for e in range(L["tile_grid"][2])], dtype=np.float64)
        else:
            c = np.full(nT, float(B))
            c[-1] = L["tokens"] - (nT - 1) * B
        M = bm.cpu().numpy().astype(np.float64)
        F = 4.0 * wl.head_dim * float(np.einsum("i,hij,j->", c, M, c))
        out[order] = {"tiles": nT, "k_per_head": kk, "attention_ms": ms,
                      "tflops": F / (ms * 1e-3) / 1e12, "flops": F}
        del ws, mb, bm, o
    out["note"] = ("top-k masks at the workload's tile density chosen on each order's tiles by the "
                   "GPU selection; attention stage of the fused forward")
    return out


def window_search(sa, wl, q, k, v, stream, tau=0.9):
    """The offline search on the workload's inputs: full-attention tile mass
    on the GPU (timed), the host search at recall tau over the temporal
    groups {0}, {1-2}, {>= 3}, and the attention stage of the fused forward
    under the searched mask."""
    import torch
    E = lambda: torch.cuda.Event(enable_timing=True)
    h = sa.sparse_attn_create(wl.heads, wl.head_dim, wl.grid, wl.tile, wl.dtype)
    L = sa.sparse_attn_layout(h)
    nT, N, d = L["tiles"], L["tokens"], wl.head_dim
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    mass = torch.empty((wl.heads, nT, nT), dtype=torch.float32, device="cuda")
    sa.sparse_attn_tile_mass(h, q, k, ws, mass)
    a, b = E(), E()
    a.record(stream)
    sa.sparse_attn_tile_mass(h, q, k, ws, mass)
    b.record(stream)
    torch.cuda.synchronize()
    mass_ms = a.elapsed_time(b)
    A = mass.cpu().numpy()
    spec = [(0, 0), (1, 2), (3, -1)]
    g_in = np.array([(lo, hi, 0, 0, 0, 0) for lo, hi in spec] * wl.heads, np.int32)
    gph = np.full(wl.heads, len(spec), np.int32)
    t0 = time.perf_counter()
    groups, rec, cost = sa.sparse_attn_search_windows(h, A, g_in, gph, tau)
    search_s = time.perf_counter() - t0
    mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_set_mask(h, mb, groups=groups, groups_per_head=gph)
    o = torch.empty_like(q)
    sa.sparse_attn_permute_kv(h, k, v, ws)
    for _ in range(2):
        sa.sparse_attn_attend_raster(h, q, o, ws)
    ev = []
    for _ in range(5):
        a, b = E(), E()
        a.record(stream)
        sa.sparse_attn_attend_raster(h, q, o, ws)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    F_mass = 2 * 2.0 * d * float(N) * float(N) * wl.heads  # two passes of Q K^T over all pairs
    F_attn = 4.0 * d * float(N) * float(N) * wl.heads * float(cost.mean())
    return {"tau": tau, "mass_ms": mass_ms, "mass_tflops": F_mass / (mass_ms * 1e-3) / 1e12,
            "search_s": search_s, "recall_mean": float(rec.mean()), "recall_min": float(rec.min()),
            "token_density_mean": float(cost.mean()), "attention_ms": attn_ms,
            "attention_tflops": F_attn / (attn_ms * 1e-3) / 1e12,
            "note": "tile mass of full attention on the GPU (both passes, with the Q/K permute), "
                    "host greedy dual-window search per head, attention stage under the searched mask"}


def copy_reference(stream, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of nbytes (torch copy_) on the same GPU:
    what a streaming read + write sustains here, as context for the HBM-bound
    permute stages' fraction of the published 8 TB/s.  Bytes counted: read
    plus written."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    gbs = 2.0 * nbytes / (ms * 1e-3) / 1e9
    return {"bytes": nbytes, "ms": ms, "gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS}


def gemm_reference(stream, n=16384, reps=5):
    """A dense bf16 library GEMM (torch.matmul, n x n x n) on the same GPU:
    what a plain matrix product sustains here under the same power and clock
    conditions, as context for the attention kernel's fraction of the
    published peak."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(2):
        c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        c = a @ b
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"shape": [n, n, n], "ms": ms, "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS}


def mix_ceiling(sa, stream, iters=3000):
    """The attention stage's instruction mix with nothing else in the way
    (sparse_attn_mix_probe: per stage and wave 32 bf16 32x32x16 products with
    operands from LDS, the kernels' online-softmax step and a barrier; no
    copies, no key lists, no global memory traffic), in the pair kernel's
    ping-pong (two synchronised waves per SIMD, half a step apart) and with
    2 (the row kernel's occupancy) and 3 unsynchronised waves per SIMD.  Reported beside the
    library GEMM as context for the attention stage's fraction of the
    published peak: the clock, and so the rate, follows the power this work
    draws.  mfma_busy counts 32 clocks per product (1024 FLOP per clock per
    SIMD at the published peak) over the slowest wave's loop, which spans
    nearly the whole launch (the waves of a SIMD do not finish together);
    clock_ghz is that wave's s_memtime cycles over the launch's event
    time; wave_cycles gives the spread."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for w, pp in ((2, True), (2, False), (3, False)):
        n = cus * w
        cyc = torch.zeros(n * 4, dtype=torch.int64, device="cuda")
        sink = torch.empty(n * 256, dtype=torch.float32, device="cuda")
        sa.sparse_attn_mix_probe(w, cus, iters, cyc, sink, pingpong=pp, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sa.sparse_attn_mix_probe(w, cus, iters, cyc, sink, pingpong=pp, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = cyc.cpu().numpy().astype(np.float64)
        span = float(c.max())
        tf = n * 4 * iters * 32 * 32768.0 / (ms * 1e-3) / 1e12
        out.append({"schedule": "ping-pong (pair kernel)" if pp else "independent waves",
                    "waves_per_simd": w, "ms": ms, "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS,
                    "wave_cycles": {"min": float(c.min()), "median": float(np.median(c)), "max": span},
                    "mfma_busy": w * 32 * 32 * iters / span, "clock_ghz": span / (ms * 1e-3) / 1e9})
        del cyc, sink
    return out


def tile_volume_sweep(sa, seed=1, reps=5):
    """Attention stage of layouts of several tile volumes on the Wan grid
    (4 heads), bf16 and fp32 on the matrix-core kernels and, for comparison,
    on the vector-ALU kernel (vector_alu = 1).  Mask: a seeded random 25%
    of the tile pairs plus the diagonal; inputs N(0, 1) rounded to the
    element type.  TFLOP/s counts real tokens only (F_alg)."""
    import torch
    from workloads import f32_to_bf16_bits

    grid, heads = (21, 45, 80), 4
    cases = [((1, 8, 16), 128, "bf16", False), ((1, 8, 16), 128, "bf16", True),
             ((1, 8, 8), 128, "bf16", False), ((1, 8, 8), 128, "bf16", True),
             ((2, 4, 8), 128, "bf16", False), ((1, 8, 8), 64, "bf16", False),
             ((1, 4, 8), 128, "bf16", False), ((1, 4, 8), 128, "bf16", True),
             ((1, 8, 16), 128, "f32", False), ((1, 8, 16), 128, "f32", True),
             ((1, 8, 8), 128, "f32", False), ((1, 8, 16), 64, "f32", False)]
    stream = torch.cuda.current_stream()
    out = []
    for tile, d, dtype, vec in cases:
        h = sa.sparse_attn_create(heads, d, grid, tile, dtype, vector_alu=vec)
        L = sa.sparse_attn_layout(h)
        nT = L["tiles"]
        rng = np.random.default_rng(seed)
        M = (rng.random((heads, nT, nT)) < 0.25).astype(np.uint8)
        M[:, np.arange(nT), np.arange(nT)] = 1
        x = rng.standard_normal((heads, int(np.prod(grid)), d), dtype=np.float32)
        xt = torch.from_numpy(f32_to_bf16_bits(x).view(np.int16) if dtype == "bf16" else x).cuda()
        mb = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
        sa.sparse_attn_set_mask(h, mb, bitmap=torch.from_numpy(M).cuda())
        ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(xt)
        sa.sparse_attn_permute_kv(h, xt, xt, ws)
        sa.sparse_attn_attend_raster(h, xt, o, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            sa.sparse_attn_attend_raster(h, xt, o, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nt, ny, nx = L["tile_grid"]
        c = np.array([min(tile[0], grid[0] - a * tile[0]) * min(tile[1], grid[1] - b * tile[1])
                      * min(tile[2], grid[2] - e * tile[2])
                      for a in range(nt) for b in range(ny) for e in range(nx)], dtype=np.float64)
        F = 4.0 * d * sum(float(c @ M[hh].astype(np.float64) @ c) for hh in range(heads))
        out.append({"tile": list(tile), "tile_volume": L["tile_volume"], "slot_stride": L["slot_stride"],
                    "head_dim": d, "dtype": dtype,
                    "kernel": "vector ALU" if L["kernel"] == sa.SPARSE_ATTN_KERNEL_GENERIC else "matrix cores",
                    "attention_ms": ms, "tflops": F / (ms * 1e-3) / 1e12})
        del ws, mb, o, xt
        sa.sparse_attn_destroy(h)
    return {"grid": list(grid), "heads": heads, "mask": "random 25% of tile pairs + diagonal", "seed": seed,
            "reps": reps, "cases": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the all-ones-mask comparison")
    ap.add_argument("--no-search", action="store_true", help="skip the window-search measurement")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the library GEMM and device-copy references")
    ap.add_argument("--no-mix-ceiling", action="store_true",
                    help="skip the instruction-mix probe (attention stage mix, no memory traffic)")
    ap.add_argument("--no-order-comparison", action="store_true",
                    help="skip the tile-box / Hilbert-order top-k comparison")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--pairing", default="auto", choices=["auto", "overlap", "all", "none"],
                    help="work split of the matrix-core path (sparse_attn_config.pairing)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="instead of the step, time the attention stage over tile volumes and kernels "
                         "and print that as the one JSON line")
    ap.add_argument("--mix-ceiling-only", action="store_true",
                    help="instead of the step, run only the instruction-mix probe (with the library GEMM "
                         "reference) and print that as the one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(heads are independent, so a multi-GPU run would shard heads with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_major_amd as sa
    from workloads import make_workload, ones_bitmap

    torch.cuda.set_device(0)
    if args.tile_sweep:
        print(json.dumps({"tile_volume_sweep": tile_volume_sweep(sa), "env": env_info()}))
        return
    if args.mix_ceiling_only:
        stream = torch.cuda.current_stream()
        print(json.dumps({"mix_ceiling": mix_ceiling(sa, stream),
                          "library_gemm_reference": gemm_reference(stream), "env": env_info()}))
        return
    wl = make_workload(args.workload)
    cfg = wl.config
    info = wl.info
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    q, k, v = t(wl.q), t(wl.k), t(wl.v)
    o = torch.empty_like(q)
    h = sa.sparse_attn_create(wl.heads, wl.head_dim, wl.grid, wl.tile, wl.dtype, pairing=args.pairing)
    ws = torch.empty(sa.sparse_attn_workspace_bytes(h), dtype=torch.uint8, device="cuda")
    mask_buf = torch.empty(sa.sparse_attn_mask_bytes(h, info["nnz"]), dtype=torch.uint8, device="cuda")
    dense_buf = torch.empty(sa.sparse_attn_mask_bytes(h), dtype=torch.uint8, device="cuda")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()
    ones = u8(ones_bitmap(wl))
    stream = torch.cuda.current_stream()

    def set_mask():
        if wl.mask_kind == "bitmap":
            sa.sparse_attn_set_mask(h, mask_buf, bitmap=u8(wl.bitmap), max_nnz=info["nnz"])
        else:
            sa.sparse_attn_set_mask(h, mask_buf, groups=wl.groups, groups_per_head=wl.groups_per_head,
                                    max_nnz=info["nnz"])

    if wl.mask_kind == "bitmap":
        bitmap_dev = u8(wl.bitmap)

        def set_mask():  # noqa: F811  (bitmap already resident)
            sa.sparse_attn_set_mask(h, mask_buf, bitmap=bitmap_dev, max_nnz=info["nnz"])

    E = lambda: torch.cuda.Event(enable_timing=True)

    # sparse_attn_forward is exactly these two stages; they are called one by
    # one so the attention launches can be timed on their own.
    def step(ev=None):
        if ev is None:
            set_mask()
            sa.sparse_attn_forward(h, q, k, v, o, ws)
            return
        ev[0].record(stream)
        set_mask()
        ev[1].record(stream)
        sa.sparse_attn_permute_kv(h, k, v, ws)
        ev[2].record(stream)
        sa.sparse_attn_attend_raster(h, q, o, ws)
        ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[E() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in events])  # ms
    mask_ms, perm_ms, attn_ms = st.mean(axis=0)
    attn_min = st[:, 2].min()
    attn_median = float(np.median(st[:, 2]))

    # The same attention launches also writing the per-query log-sum-exp.
    lse = torch.empty((wl.heads, cfg.tokens), dtype=torch.float32, device="cuda")
    sa.sparse_attn_attend_raster(h, q, o, ws, lse=lse)
    lse_ev = []
    for _ in range(5):
        a, b = E(), E()
        a.record(stream)
        sa.sparse_attn_attend_raster(h, q, o, ws, lse=lse)
        b.record(stream)
        lse_ev.append((a, b))
    torch.cuda.synchronize()
    attn_lse_ms = float(np.mean([a.elapsed_time(b) for a, b in lse_ev]))
    del lse

    # The standalone unpermute of the three-stage path (the step fuses it
    # into the attention epilogue).
    sa.sparse_attn_permute_inputs(h, q, k, v, ws)
    sa.sparse_attn_attend(h, ws)
    sa.sparse_attn_unpermute_output(h, ws, o)
    unp = []
    for _ in range(5):
        a, b = E(), E()
        a.record(stream)
        sa.sparse_attn_unpermute_output(h, ws, o)
        b.record(stream)
        unp.append((a, b))
    torch.cuda.synchronize()
    unperm_ms = float(np.mean([a.elapsed_time(b) for a, b in unp]))
    nnz, overflow = sa.sparse_attn_mask_info(h)
    assert nnz == info["nnz"] and not overflow, (nnz, info["nnz"], overflow)

    # Same kernel, same inputs, all-ones mask.
    dense_ms = None
    if not args.no_dense:
        sa.sparse_attn_set_mask(h, dense_buf, bitmap=ones)
        sa.sparse_attn_permute_kv(h, k, v, ws)
        for _ in range(2):
            sa.sparse_attn_attend_raster(h, q, o, ws)
        dense = []
        for _ in range(max(3, args.steps // 4)):
            a, b = E(), E()
            a.record(stream)
            sa.sparse_attn_attend_raster(h, q, o, ws)
            b.record(stream)
            dense.append((a, b))
        torch.cuda.synchronize()
        dense_ms = float(np.mean([a.elapsed_time(b) for a, b in dense]))

    # Tile selection (the step that chooses top-k masks from Q and K; not part
    # of the timed step): k per head from the workload when it is a top-k
    # workload, else the workload's tile density.
    nT = info["nT"]
    kh = info.get("k_per_head") or [max(1, round(info["tile_density"] * nT))] * wl.heads
    sel_bitmap = torch.empty((wl.heads, nT, nT), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_permute_inputs(h, q, k, v, ws)
    sa.sparse_attn_select_topk(h, kh, ws, sel_bitmap)
    sel = []
    for _ in range(5):
        a, b = E(), E()
        a.record(stream)
        sa.sparse_attn_select_topk(h, kh, ws, sel_bitmap)
        b.record(stream)
        sel.append((a, b))
    torch.cuda.synchronize()
    select_ms = float(np.mean([a.elapsed_time(b) for a, b in sel]))
    # The same with the per-head Top-k estimate (Top-p 0.9, fixed floor of a
    # tenth of the key tiles, the page's ratio).
    scope_keep = torch.empty((wl.heads, nT), dtype=torch.int32, device="cuda")
    rho, k_fixed = 0.9, -(-nT // 10)
    sa.sparse_attn_select_scope(h, rho, k_fixed, ws, sel_bitmap, keep=scope_keep)
    sel = []
    for _ in range(5):
        a, b = E(), E()
        a.record(stream)
        sa.sparse_attn_select_scope(h, rho, k_fixed, ws, sel_bitmap, keep=scope_keep)
        b.record(stream)
        sel.append((a, b))
    torch.cuda.synchronize()
    scope_ms = float(np.mean([a.elapsed_time(b) for a, b in sel]))
    scope_keep_mean = float(scope_keep.double().mean())
    del sel_bitmap, scope_keep

    gemm = None if args.no_gemm_reference else gemm_reference(stream)
    copy_ref = None if args.no_gemm_reference else copy_reference(stream)
    mix = None if args.no_mix_ceiling else mix_ceiling(sa, stream)
    searched = None
    if not args.no_search:
        searched = window_search(sa, wl, q, k, v, stream)
    orders = None
    if not args.no_order_comparison:
        orders = topk_order_comparison(sa, wl, q, k, v, info["tile_density"], stream)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    F = info["flops_alg"]
    N, d, heads = cfg.tokens, cfg.head_dim, wl.heads
    elem = 2
    attn_tflops = F / (attn_ms * 1e-3) / 1e12
    in_bytes = heads * N * d * elem
    slot_bytes = heads * sa.sparse_attn_layout(h)["slots"] * d * elem
    perm_bytes = 2 * (in_bytes + slot_bytes)  # K and V: raster read, tile-major written
    # The counter profile is taken with the default work split.
    traffic = traffic_per_launch(args.workload) if args.pairing == "auto" else None
    result = {
        "metric": METRIC,
        "value": F / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "heads": heads, "head_dim": d,
                   "grid": list(cfg.grid), "tile": list(cfg.tile), "tokens": N,
                   "tile_density": round(info["tile_density"], 5),
                   "token_density": round(info["token_density"], 5),
                   "pairing": args.pairing,
                   "step": "mask compile + permute K, V + block-sparse attention (Q read and O "
                           "written in raster order by the attention kernels)",
                   "inputs": input_fingerprint(wl)},
        "roofline": {"bound": "mfma", "kernel": ATTN_KERNELS, "achieved": attn_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "flops_per_launch": F,
                     "library_gemm_reference": gemm, "mix_ceiling": mix,
                     # the attention stage's rate over that of the instruction-mix probe in
                     # the pair kernel's own schedule (no copies, lists or clipped tiles)
                     "frac_of_pingpong_mix": (attn_tflops / mix[0]["tflops"]) if mix else None},
        "attention": {"ms": attn_ms, "ms_median": attn_median, "ms_min": float(attn_min),
                      "tflops": attn_tflops,
                      "pct_peak": 100 * attn_tflops / PEAK_BF16_TFLOPS,
                      # as if every kept tile pair were a full B x B block (the kernels
                      # skip padding at 32-key / 32-query granularity; the MFMA counters
                      # give their issued work)
                      "tflops_full_tiles": info["flops_issued"] / (attn_ms * 1e-3) / 1e12,
                      "dense_ms": dense_ms,
                      "dense_speedup": dense_ms / attn_ms if dense_ms else None,
                      "ideal_speedup": info["flops_dense"] / F,
                      "dense_tflops": info["flops_dense"] / (dense_ms * 1e-3) / 1e12 if dense_ms else None,
                      "with_lse_ms": attn_lse_ms},
        "stages_ms": {"mask_compile": mask_ms, "permute_kv": perm_ms, "attention": attn_ms},
        "stages_gbs": {"permute_kv": perm_bytes / (perm_ms * 1e-3) / 1e9,
                       "unpermute_o_standalone": 2 * in_bytes / (unperm_ms * 1e-3) / 1e9,
                       "mask_compile": mask_buf.numel() / (mask_ms * 1e-3) / 1e9,
                       "peak": PEAK_HBM_GBS,
                       "device_copy_reference": copy_ref,
                       "note": "unpermute: real rows read + written, timed outside the step (the step "
                               "fuses it); mask compile: bytes of the compiled-mask buffer per call, "
                               "a launch- and latency-bound integer stage"},
        "unpermute_o_standalone_ms": unperm_ms,
        "tile_selection": {"ms": select_ms, "k_per_head": [int(x) for x in kh],
                           "pool_gbs": 2 * in_bytes / (select_ms * 1e-3) / 1e9,
                           "note": "top-k over mean-pooled tile scores from the permuted Q, K; "
                                   "not part of the timed step",
                           "per_head_estimate": {"ms": scope_ms, "rho": rho, "k_fixed": k_fixed,
                                                 "mean_tiles_kept": scope_keep_mean}},
        "topk_by_token_order": orders,
        "window_search": searched,
        "env": env_info(),
    }
    if not args.no_cpu_baseline:
        import oracle
        M = oracle.mask_of(wl)
        result["cpu_baseline"] = cpu_baseline(wl, M)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def env_info():
    """Device and software the numbers were taken on."""
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "memory_gb": round(props.total_memory / 2 ** 30, 1),
            "hip": torch.version.hip, "torch": torch.__version__}


if __name__ == "__main__":
    main()

"""Seeded synthetic workloads for tile-masked video attention.

Five workloads stand in for the attention inputs of video diffusion
transformers at their real shapes (the pages evaluate Wan2.1-14B and
HunyuanVideo at 720p on Open-Sora/VBench prompts, which are not available
here, so Q/K/V are synthetic):

  tiny      2 heads, d=64, fp32, grid 4x8x8, tile 1x4x4, Bernoulli(0.5) tile
            mask with the diagonal tile kept
  small    12 heads, d=128, bf16, grid 8x30x40, tile 1x8x16, dual-window
            spec over 3 temporal-distance groups, shrunk to <= 30% density
  wan      40 heads, d=128, bf16, grid 21x45x80 (75,600 tokens), tile
            1x8x16, Q/K with a shared low-rank spatial bias, local / axial /
            near-dense heads, overall tile density in [23.5%, 26.5%]
  hunyuan  24 heads, d=128, bf16, grid 33x45x80 (118,800 tokens), tile
            1x8x16, per-head top-k over mean-pooled tile scores
  long     40 heads, d=128, bf16, grid 42x45x80 (151,200 tokens), tile
            1x8x16, +-4 frames and one axial window, about 10% density

Everything is drawn with numpy PCG64 from ``default_rng([1000 + index,
stream, ...])`` with stream 0 = Q, 1 = K, 2 = V, 3 = mask, 4 = bias, and a
per-head sub-seed, so any prefix of the heads is identical to the same heads
of the full workload.

The dual-window reading used by the mask recipes (Compact Attention page,
Fig. 1 caption part (3) and Fig. 4 caption): per head, temporal-distance
groups [dt_lo, dt_hi] in tile units along t (dt_hi = -1: unbounded), each
with two rectangular windows given by symmetric half-extents (ry, rx) in
tiles around the query tile; -1 disables a window.  This module only draws
the specs; evaluating them into masks is done separately by the oracle and
by the GPU mask compiler.

This module holds the input recipes only.  Counting formulas used to steer
the recipes towards their density targets live in ``accounting``.
"""

import concurrent.futures
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import accounting
from .bf16 import f32_to_bf16_bits


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    grid: tuple  # (T, H, W)
    tile: tuple  # (tt, th, tw)
    mask: str  # recipe name

    @property
    def seed(self):
        return 1000 + self.index

    @property
    def tokens(self):
        T, H, W = self.grid
        return T * H * W


CONFIGS = {
    "tiny": Config("tiny", 0, 2, 64, "f32", (4, 8, 8), (1, 4, 4), "bernoulli"),
    "small": Config("small", 1, 12, 128, "bf16", (8, 30, 40), (1, 8, 16), "small_windows"),
    "wan": Config("wan", 2, 40, 128, "bf16", (21, 45, 80), (1, 8, 16), "wan_windows"),
    "hunyuan": Config("hunyuan", 3, 24, 128, "bf16", (33, 45, 80), (1, 8, 16), "hunyuan_topk"),
    "long": Config("long", 4, 40, 128, "bf16", (42, 45, 80), (1, 8, 16), "long_axial"),
}

# Temporal-distance groups shared by the small and wan recipes: |dt| = 0,
# 1..2 and >= 3 (tile units along t; tt = 1 so these are frames).
THREE_GROUPS = ((0, 0), (1, 2), (3, -1))


@dataclass
class Workload:
    config: Config
    heads: int
    q: np.ndarray  # [heads, N, d] float32, or uint16 bf16 bit patterns
    k: np.ndarray
    v: np.ndarray
    mask_kind: str  # "bitmap" or "windows"
    bitmap: Optional[np.ndarray] = None  # uint8 [heads, nT, nT], nonzero = keep
    groups: Optional[np.ndarray] = None  # int32 [G, 6]: dt_lo, dt_hi, ry0, ry1, rx0, rx1
    groups_per_head: Optional[np.ndarray] = None  # int32 [heads]
    info: dict = field(default_factory=dict)

    @property
    def grid(self):
        return self.config.grid

    @property
    def tile(self):
        return self.config.tile

    @property
    def head_dim(self):
        return self.config.head_dim

    @property
    def dtype(self):
        return self.config.dtype


def tile_grid(grid, tile):
    """Number of tiles along (t, y, x) for a grid cut into tiles (ceil)."""
    return tuple(-(-g // t) for g, t in zip(grid, tile))


def _rng(cfg, stream, *sub):
    return np.random.default_rng([cfg.seed, stream, *sub])


def _encode(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _per_head(heads, fn):
    """Run fn(h) for every head on a thread pool (numpy releases the GIL in
    the RNG and array kernels); each head has its own seeded stream, so the
    result does not depend on scheduling."""
    workers = max(1, min(16, len(os.sched_getaffinity(0)), heads))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fn, range(heads)))


def _gaussian(cfg, stream, heads):
    N, d = cfg.tokens, cfg.head_dim
    out = np.empty((heads, N, d), dtype=np.float32 if cfg.dtype == "f32" else np.uint16)

    def one(h):
        out[h] = _encode(_rng(cfg, stream, h).standard_normal((N, d), dtype=np.float32), cfg.dtype)

    _per_head(heads, one)
    return out


# ----------------------------------------------------------------------------
# Mask recipes


def _bernoulli_bitmap(cfg, heads):
    nT = int(np.prod(tile_grid(cfg.grid, cfg.tile)))
    M = np.empty((heads, nT, nT), dtype=np.uint8)
    for h in range(heads):
        M[h] = _rng(cfg, 3, h).random((nT, nT)) < 0.5
        np.fill_diagonal(M[h], 1)
    return M


def _pack_groups(per_head):
    """per_head: list over heads of lists of (dt_lo, dt_hi, ry0, ry1, rx0, rx1)."""
    gph = np.array([len(g) for g in per_head], dtype=np.int32)
    rows = [row for g in per_head for row in g]
    return np.array(rows, dtype=np.int32).reshape(-1, 6), gph


def _small_windows(cfg):
    """Two windows per group with half-extents drawn from U{0..4} (clamped to
    the tile grid), then shrunk round-robin over heads until the overall tile
    density is at most 30%.  The shrink move is the one the Compact Attention
    page describes for its offline search (Fig. 3 and Fig. 4 captions: the
    dual windows are shrunk step by step); here it only steers a random draw
    towards the density target."""
    nt, ny, nx = tile_grid(cfg.grid, cfg.tile)
    rng = _rng(cfg, 3)
    heads = []
    for _h in range(cfg.heads):
        groups = []
        for lo, hi in THREE_GROUPS:
            w = rng.integers(0, 5, size=(2, 2))  # [window][axis y, x]
            groups.append([lo, hi, min(w[0, 0], ny - 1), min(w[1, 0], ny - 1),
                           min(w[0, 1], nx - 1), min(w[1, 1], nx - 1)])
        heads.append(groups)

    def density():
        return accounting.window_nnz_total(heads, (nt, ny, nx)) / (cfg.heads * (nt * ny * nx) ** 2)

    def shrink(groups):
        # Farthest group holding a window that may still shrink.
        for g in range(len(groups) - 1, -1, -1):
            lo, hi, ry0, ry1, rx0, rx1 = groups[g]
            cands = []
            for w, (ry, rx) in enumerate(((ry0, rx0), (ry1, rx1))):
                if ry < 0 or rx < 0:
                    continue
                if g == 0 and w == 0 and ry == 0 and rx == 0:
                    continue  # the diagonal window stays
                cands.append(((2 * ry + 1) * (2 * rx + 1), -w, w, ry, rx))
            if not cands:
                continue
            _, _, w, ry, rx = max(cands)
            if ry == 0 and rx == 0:
                ry, rx = -1, -1
            elif ry >= rx:
                ry -= 1
            else:
                rx -= 1
            groups[g][2 + w] = ry
            groups[g][4 + w] = rx
            return True
        return False

    h = 0
    stuck = 0
    while density() > 0.30 and stuck < cfg.heads:
        stuck = 0 if shrink(heads[h]) else stuck + 1
        h = (h + 1) % cfg.heads
    return heads


def _wan_windows(cfg):
    """Heads by h mod 3: local, axial, near-dense (Compact Attention page,
    Fig. 1 caption part (2): heads show local, axial or dense coarse
    regions).  The first draw whose overall tile density lies in
    [23.5%, 26.5%] is kept."""
    nt, ny, nx = tile_grid(cfg.grid, cfg.tile)
    fy, fx = ny - 1, nx - 1
    for attempt in range(1000):
        heads = []
        for h in range(cfg.heads):
            rng = _rng(cfg, 3, attempt, h)
            kind = h % 3
            if kind == 0:  # local
                a = rng.integers(0, 3, size=4)
                b = rng.integers(0, 2, size=4)
                groups = [[0, 0, a[0], a[1], a[2], a[3]],
                          [1, 2, b[0], b[1], b[2], b[3]],
                          [3, -1, -1, -1, -1, -1]]
            elif kind == 1:  # axial: a row band and a column band
                a, b = rng.integers(0, 2, size=2)
                groups = [[0, 0, a, fy, fx, b],
                          [1, 2, a, fy, fx, b],
                          [3, -1, -1, -1, -1, -1]]
            else:  # near-dense
                ry = rng.integers(1, 4, size=2)
                rx = rng.integers(1, 3, size=2)
                groups = [[0, 0, fy, -1, fx, -1],
                          [1, 2, fy, -1, fx, -1],
                          [3, -1, ry[0], ry[1], rx[0], rx[1]]]
            heads.append([[int(x) for x in g] for g in groups])
        dens = accounting.window_nnz_total(heads, (nt, ny, nx)) / (cfg.heads * (nt * ny * nx) ** 2)
        if 0.235 <= dens <= 0.265:
            return heads, attempt
    raise RuntimeError("wan mask recipe found no draw in its density band")


def _long_windows(cfg):
    """One temporal group |dt| <= 4 and one axial window per head: a row band
    (ry = r, rx = full) or a column band (ry = full, rx = r), r ~ U{0,1,2}."""
    nt, ny, nx = tile_grid(cfg.grid, cfg.tile)
    heads = []
    for h in range(cfg.heads):
        rng = _rng(cfg, 3, h)
        row = rng.random() < 0.5
        r = int(rng.integers(0, 3))
        ry, rx = (r, nx - 1) if row else (ny - 1, r)
        heads.append([[0, 4, ry, -1, rx, -1]])
    return heads


def _tile_means(x, grid, tile):
    """fp64 mean of each tile's real tokens: x [N, d] -> [nT, d]."""
    T, H, W = grid
    tt, th, tw = tile
    nt, ny, nx = tile_grid(grid, tile)
    d = x.shape[-1]
    g = np.zeros((nt * tt, ny * th, nx * tw, d), dtype=np.float64)
    g[:T, :H, :W] = x.reshape(T, H, W, d)
    ones = np.zeros((nt * tt, ny * th, nx * tw), dtype=np.float64)
    ones[:T, :H, :W] = 1.0
    s = g.reshape(nt, tt, ny, th, nx, tw, d).sum(axis=(1, 3, 5))
    c = ones.reshape(nt, tt, ny, th, nx, tw).sum(axis=(1, 3, 5))
    return (s / c[..., None]).reshape(nt * ny * nx, d)


def _hunyuan_topk(cfg, q, k, heads):
    """Row i keeps the k_h key tiles with the largest mean-pooled score
    qbar_i . kbar_j / sqrt(d) (ties to the lower j), k_h = round(u_h * nT)
    with u_h ~ U(0.10, 0.40).  Block-level proxy scoring as named on the
    SCOPE review page (abstract) and the AdaSpa page (blockified pattern)."""
    nT = int(np.prod(tile_grid(cfg.grid, cfg.tile)))
    M = np.zeros((heads, nT, nT), dtype=np.uint8)
    ks = []
    for h in range(heads):
        u = _rng(cfg, 3, h).uniform(0.10, 0.40)
        kh = int(min(max(int(np.floor(u * nT + 0.5)), 1), nT))
        ks.append(kh)
        qf = q[h].astype(np.float32) if cfg.dtype == "f32" else (q[h].astype(np.uint32) << 16).view(np.float32)
        kf = k[h].astype(np.float32) if cfg.dtype == "f32" else (k[h].astype(np.uint32) << 16).view(np.float32)
        qb = _tile_means(qf, cfg.grid, cfg.tile)
        kb = _tile_means(kf, cfg.grid, cfg.tile)
        S = qb @ kb.T / np.sqrt(cfg.head_dim)
        idx = np.argsort(-S, axis=1, kind="stable")[:, :kh]
        np.put_along_axis(M[h], idx, 1, axis=1)
    return M, ks


# ----------------------------------------------------------------------------
# Q/K/V recipes


def _wan_qk(cfg, stream, heads):
    """q = alpha (z + beta phi(p) U_h): z ~ N(0, 1), phi a 16-dim random
    Fourier feature of the token position (t, y, x) with length scales
    (1.5, 6, 12) tokens, U_h a per-head 16 x d orthonormal map.  beta^2 =
    4 sqrt(d) / (1 - 4 / sqrt(d)) puts a +4 peak on the scaled score at zero
    offset and alpha = (1 + beta^2 / d)^(-1/2) keeps unit element variance."""
    T, H, W = cfg.grid
    d = cfg.head_dim
    beta2 = 4.0 * np.sqrt(d) / (1.0 - 4.0 / np.sqrt(d))
    beta = np.sqrt(beta2)
    alpha = 1.0 / np.sqrt(1.0 + beta2 / d)
    omega = _rng(cfg, 4).standard_normal((8, 3)) / np.array([1.5, 6.0, 12.0])
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    p = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)
    ang = p @ omega.T
    phi = (np.concatenate([np.cos(ang), np.sin(ang)], axis=1) / np.sqrt(8.0)).astype(np.float32)
    out = np.empty((heads, cfg.tokens, d), dtype=np.uint16)

    def one(h):
        u, _ = np.linalg.qr(_rng(cfg, 4, h + 1).standard_normal((d, 16)))
        bias = phi @ u.T.astype(np.float32)
        z = _rng(cfg, stream, h).standard_normal((cfg.tokens, d), dtype=np.float32)
        out[h] = _encode(np.float32(alpha) * (z + np.float32(beta) * bias), cfg.dtype)

    _per_head(heads, one)
    return out


def make_workload(name, heads=None, masks_only=False):
    """Build the named workload; ``heads`` limits generation to the first
    heads (identical to those heads of the full workload).  ``masks_only``
    skips drawing Q/K/V when the mask recipe does not need them (q, k, v are
    then None)."""
    cfg = CONFIGS[name]
    heads = cfg.heads if heads is None else int(heads)
    if not 1 <= heads <= cfg.heads:
        raise ValueError(f"heads must be in 1..{cfg.heads}")
    info = {}
    if masks_only and cfg.mask != "hunyuan_topk":
        q = k = v = None
    elif cfg.mask == "wan_windows":
        q, k = _wan_qk(cfg, 0, heads), _wan_qk(cfg, 1, heads)
        v = _gaussian(cfg, 2, heads)
    else:
        q, k = _gaussian(cfg, 0, heads), _gaussian(cfg, 1, heads)
        v = None if masks_only else _gaussian(cfg, 2, heads)

    if cfg.mask == "bernoulli":
        wl = Workload(cfg, heads, q, k, v, "bitmap", bitmap=_bernoulli_bitmap(cfg, heads))
    elif cfg.mask == "hunyuan_topk":
        M, ks = _hunyuan_topk(cfg, q, k, heads)
        info["k_per_head"] = ks
        wl = Workload(cfg, heads, q, k, v, "bitmap", bitmap=M)
    else:
        if cfg.mask == "small_windows":
            per_head = _small_windows(cfg)
        elif cfg.mask == "wan_windows":
            per_head, attempt = _wan_windows(cfg)
            info["mask_attempt"] = attempt
        else:
            per_head = _long_windows(cfg)
        groups, gph = _pack_groups(per_head[:heads])
        wl = Workload(cfg, heads, q, k, v, "windows", groups=groups, groups_per_head=gph)
    wl.info.update(info)
    wl.info.update(accounting.summarize(wl))
    return wl


def ones_bitmap(wl):
    """The all-ones tile mask for a workload (the dense-mask variant)."""
    nT = int(np.prod(tile_grid(wl.grid, wl.tile)))
    return np.ones((wl.heads, nT, nT), dtype=np.uint8)

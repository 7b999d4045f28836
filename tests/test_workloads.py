"""The synthetic workload recipes: determinism, shapes and density bands."""

import numpy as np
import pytest

from workloads import CONFIGS, accounting, bf16_bits_to_f32, f32_to_bf16_bits, make_workload
from workloads.configs import _long_windows, _wan_windows, tile_grid


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, np.inf, 1e-40], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1); 1 + 3 * 2^-8 -> 1 + 2^-6
    assert got.tolist()[:5] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0]
    assert np.isinf(got[5]) and np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.float32([np.nan]))))[0]


def test_tiny_is_deterministic_and_keeps_the_diagonal():
    a, b = make_workload("tiny"), make_workload("tiny")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.bitmap, b.bitmap)
    assert a.q.dtype == np.float32 and a.q.shape == (2, 256, 64)
    for h in range(2):
        assert np.all(np.diag(a.bitmap[h]) == 1)
    assert 0.45 < a.info["tile_density"] < 0.6


def test_small_density_and_groups():
    wl = make_workload("small")
    assert wl.q.dtype == np.uint16 and wl.q.shape == (12, 9600, 128)
    assert 0.27 <= wl.info["tile_density"] <= 0.30
    assert np.all(wl.groups_per_head == 3)
    g = wl.groups.reshape(12, 3, 6)
    assert np.all(g[:, 0, 2] >= 0) and np.all(g[:, 0, 4] >= 0)  # diagonal window kept


def test_head_prefix_matches_full_workload():
    a = make_workload("small", heads=3)
    b = make_workload("small")
    assert np.array_equal(a.q, b.q[:3]) and np.array_equal(a.groups, b.groups[:9])


def test_wan_mask_mix_and_band():
    cfg = CONFIGS["wan"]
    per_head, _ = _wan_windows(cfg)
    tg = tile_grid(cfg.grid, cfg.tile)
    nT = int(np.prod(tg))
    dens = [accounting.window_nnz(g, tg) / nT ** 2 for g in per_head]
    assert 0.235 <= np.mean(dens) <= 0.265
    local, axial, dense = dens[0::3], dens[1::3], dens[2::3]
    assert len(local) == 14 and len(axial) == 13 and len(dense) == 13
    assert max(local) < min(dense) and np.mean(local) < np.mean(axial) < np.mean(dense)


def test_wan_bias_concentrates_scores_locally():
    wl = make_workload("wan", heads=1)
    q = bf16_bits_to_f32(wl.q[0]).astype(np.float64)
    k = bf16_bits_to_f32(wl.k[0]).astype(np.float64)
    assert abs(q.var() - 1.0) < 0.05 and abs(k.var() - 1.0) < 0.05
    # same-position score is lifted by about +4 on average
    s_same = np.einsum("nd,nd->n", q[:2000], k[:2000]) / np.sqrt(128)
    s_far = np.einsum("nd,nd->n", q[:2000], k[-2000:]) / np.sqrt(128)
    assert 3.0 < s_same.mean() < 5.0 and abs(s_far.mean()) < 1.5


def test_long_density():
    cfg = CONFIGS["long"]
    tg = tile_grid(cfg.grid, cfg.tile)
    nnz = accounting.window_nnz_total(_long_windows(cfg), tg)
    assert 0.07 < nnz / (cfg.heads * np.prod(tg) ** 2) < 0.13


def test_hunyuan_rows_keep_exactly_k():
    wl = make_workload("hunyuan", heads=2)
    for h, kh in enumerate(wl.info["k_per_head"]):
        assert 99 <= kh <= 396
        assert np.all(wl.bitmap[h].sum(axis=1) == kh)


def test_flop_convention_matches_the_adaspa_budget():
    # AdaSpa page, abstract: an 8-second 720p HunyuanVideo clip (about 110K
    # tokens) costs about 500 PFLOP of attention.  With 4 N^2 d per head and
    # layer, 24 heads, d = 128, 60 blocks and 50 steps (model facts from
    # outside the pages) the convention lands in that range.
    per = 4.0 * 110e3 ** 2 * 128 * 24
    total = per * 60 * 50 / 1e15
    assert 400 < total < 600
    cfg = CONFIGS["tiny"]
    wl = make_workload("tiny")
    M1 = np.ones_like(wl.bitmap)
    wl.bitmap = M1
    s = accounting.summarize(wl)
    assert s["flops_alg"] == s["flops_dense"] == 4.0 * 256 ** 2 * 64 * cfg.heads

"""Host-side figures of bench.py checked on the CPU: the per-launch
algorithmic bytes follow the stated per-slot, per-face and per-vertex costs,
and the pair counts behind the fp32-VALU fraction (pixel centres inside a
live face's box grown by the blur radius, and the candidate pairs among
them) agree with an independent count: the box pairs by counting pixel
centres against each box, the candidates with the oracle, run in binary64
with K large enough to keep every candidate of every pixel."""

import numpy as np
import pytest

import bench
from workloads import make_workload


def test_algorithmic_bytes_follow_the_per_unit_costs():
    w = make_workload("small_hetero")
    b = bench.algorithmic_bytes(w, filled_slots=1000)
    assert b["fine_raster"] == 28 * w.slots + 24 * w.F + 12 * w.V
    per_filled = (4 if "zbuf" in w.grads else 0) + (12 if "bary" in w.grads else 0) + (4 if "dists" in w.grads else 0)
    assert b["backward_slots"] == 8 * w.slots + per_filled * 1000 + 24 * w.F + 24 * w.V


def _box_pairs_by_centres(w):
    """Pixel centres inside each live face's box grown by the blur radius,
    counted by comparing the centres with the box (no index arithmetic)."""
    v = w.verts.astype(np.float64)
    tri = v[w.faces]
    x, y, z = tri[..., 0], tri[..., 1], tri[..., 2]
    A = (x[:, 1] - x[:, 0]) * (y[:, 2] - y[:, 0]) - (y[:, 1] - y[:, 0]) * (x[:, 2] - x[:, 0])
    live = (A != 0) & (z.max(axis=1) > 0)
    r = np.sqrt(np.float64(w.blur))
    cx = (2.0 * np.arange(w.W) + 1.0) / w.W - 1.0
    cy = (2.0 * np.arange(w.H) + 1.0) / w.H - 1.0
    nx = np.searchsorted(cx, x.max(1) + r, side="right") - np.searchsorted(cx, x.min(1) - r, side="left")
    ny = np.searchsorted(cy, y.max(1) + r, side="right") - np.searchsorted(cy, y.min(1) - r, side="left")
    return int(np.where(live, nx * ny, 0).sum())


@pytest.mark.parametrize("name", ["small_hetero", "small_soups", "sphere64"])
def test_pair_counts_match_independent_counts(oracle_mod, name):
    w = make_workload(name)
    p_bbox, p_acc = bench.pair_counts(w, sample_pairs=1 << 40)   # every face: exact
    assert p_bbox == _box_pairs_by_centres(w)
    kmax = 64
    p2f = oracle_mod.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, kmax, w.blur, precision="f64")[0]
    per_pixel = (p2f >= 0).sum(-1)
    assert per_pixel.max() < kmax, "K too small to keep every candidate"
    cand = int(per_pixel.sum())
    # both sides decide in binary64; they may differ only at pairs that sit
    # on a decision boundary
    assert abs(p_acc - cand) <= 1e-4 * cand + 2, (p_acc, cand)
    assert p_acc <= p_bbox


def test_sampled_pair_count_is_close_to_the_exact_one():
    w = make_workload("small_hetero")
    exact = bench.pair_counts(w, sample_pairs=1 << 40)
    sampled = bench.pair_counts(w, sample_pairs=200_000, seed=7)
    assert sampled[0] == exact[0]
    assert abs(sampled[1] - exact[1]) <= 0.03 * exact[1]

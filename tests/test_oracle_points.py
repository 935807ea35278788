"""Pins of the point-cloud oracle (oracle/points.py): a hand-worked case with
the strict radius test and a depth tie, exact rational brute force on dyadic
inputs, invariants (cloud concatenation, point permutation, the prefix
property over K), and central finite differences of the backward pass."""

from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle.points import rasterize_points, rasterize_points_backward
from workloads import make_point_workload


def test_hand_case():
    # 4x4 image: pixel (1, 1) has its centre at (-0.25, -0.25); radius 0.5
    pts = np.array([[-0.25, -0.25, 2.0],    # on pixel (1, 1)'s centre
                    [-0.25, -0.25, 2.0],    # the same point again: tie on z, index decides
                    [0.25, 0.75, 1.0],      # on pixel (3, 2)'s centre
                    [0.0, 0.0, -1.0]])      # behind the camera: never a candidate
    idx, zb, ds = rasterize_points(pts, [0, 4], 4, 4, 3, 0.5)
    np.testing.assert_array_equal(idx[0, 1, 1], [0, 1, -1])
    np.testing.assert_array_equal(zb[0, 1, 1], [2.0, 2.0, -1.0])
    np.testing.assert_array_equal(ds[0, 1, 1], [0.0, 0.0, -1.0])
    # pixel (1, 2) (centre (0.25, -0.25)) is at distance 0.5 = radius from the
    # first two points: excluded (strict); pixel (2, 2) at squared distance 0.5
    assert (idx[0, 1, 2] == -1).all() and (idx[0, 2, 2] == -1).all()
    # pixel (2, 2) (centre (0.25, 0.25)) is 0.5 from point 2 as well: excluded;
    # pixel (3, 2) holds point 2 at distance 0 and pixel (3, 1) at d2 = 0.25 - excluded
    np.testing.assert_array_equal(idx[0, 3, 2], [2, -1, -1])
    assert (idx[0, 3, 1] == -1).all()
    assert not (idx == 3).any()


def _dyadic_case(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 4))
    sizes = rng.integers(0, 40, N)
    pts = np.stack([rng.integers(-70, 71, sizes.sum()) / 64.0, rng.integers(-70, 71, sizes.sum()) / 64.0,
                    rng.integers(-8, 64, sizes.sum()) / 16.0], axis=1)
    off = np.concatenate([[0], np.cumsum(sizes)])
    H, W = int(rng.choice([4, 8, 16])), int(rng.choice([4, 8, 16]))
    K = int(rng.integers(1, 6))
    radius = float(rng.choice([0.125, 0.25, 0.375]))
    return pts, off, H, W, K, radius


@pytest.mark.parametrize("seed", range(10))
def test_exact_brute_force(seed):
    pts, off, H, W, K, radius = _dyadic_case(seed)
    idx, zb, ds = rasterize_points(pts, off, H, W, K, radius)
    r2 = Fr(radius) ** 2
    for n in range(len(off) - 1):
        for i in range(H):
            for j in range(W):
                px, py = Fr(2 * j + 1, W) - 1, Fr(2 * i + 1, H) - 1
                cand = []
                for q in range(off[n], off[n + 1]):
                    x, y, z = (Fr(float(c)) for c in pts[q])
                    d2 = (px - x) ** 2 + (py - y) ** 2
                    if z > 0 and d2 < r2:
                        cand.append((z, q, d2))
                cand.sort()
                want = cand[:K]
                got = idx[n, i, j]
                assert [q for _, q, _ in want] == [int(q) for q in got if q >= 0]
                for k, (z, q, d2) in enumerate(want):
                    assert Fr(float(zb[n, i, j, k])) == z and Fr(float(ds[n, i, j, k])) == d2
                assert (got[len(want):] == -1).all()


def test_clouds_are_independent_and_k_prefix():
    w = make_point_workload("points_soup")
    full = rasterize_points(w.points, w.offsets, w.H, w.W, w.K, w.radius)
    for n in range(w.N):
        lo, hi = w.offsets[n], w.offsets[n + 1]
        one = rasterize_points(w.points[lo:hi], [0, hi - lo], w.H, w.W, w.K, w.radius)
        shifted = np.where(one[0] >= 0, one[0] + lo, -1)
        np.testing.assert_array_equal(shifted[0], full[0][n])
        np.testing.assert_array_equal(one[1][0], full[1][n])
        np.testing.assert_array_equal(one[2][0], full[2][n])
    k3 = rasterize_points(w.points, w.offsets, w.H, w.W, 3, w.radius)
    for a, b in zip(k3, full):
        np.testing.assert_array_equal(a, b[..., :3])


def test_point_permutation():
    w = make_point_workload("points_small")
    pts = w.points.copy()
    pts[:, 2] += np.random.default_rng(0).uniform(0, 1e-3, len(pts)).astype(np.float32)   # distinct depths
    ref = rasterize_points(pts, w.offsets, w.H, w.W, w.K, w.radius)
    perm = np.arange(len(pts))
    for n in range(w.N):
        lo, hi = w.offsets[n], w.offsets[n + 1]
        perm[lo:hi] = lo + np.random.default_rng(n).permutation(hi - lo)
    got = rasterize_points(pts[perm], w.offsets, w.H, w.W, w.K, w.radius)
    np.testing.assert_array_equal(np.where(got[0] >= 0, perm[got[0]], -1), ref[0])
    np.testing.assert_array_equal(got[1], ref[1])
    np.testing.assert_array_equal(got[2], ref[2])


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(seed)
    P, H, W, K, radius = 12, 12, 12, 3, 0.3
    pts = np.concatenate([rng.uniform(-0.8, 0.8, (P, 2)), rng.uniform(0.5, 2.0, (P, 1))], axis=1)
    off = [0, 7, P]
    gz = rng.normal(size=(2, H, W, K))
    gd = rng.normal(size=(2, H, W, K))
    idx, _, _ = rasterize_points(pts, off, H, W, K, radius, precision="f64")
    grad = rasterize_points_backward(pts, off, H, W, K, idx, gz, gd, precision="f64")

    def loss(p):
        i, z, d = rasterize_points(p, off, H, W, K, radius, precision="f64")
        return float((gz * z).sum() + (gd * d).sum()), i

    h = 1e-7
    tested = 0
    for q in range(P):
        for c in range(3):
            pp, pm = pts.copy(), pts.copy()
            pp[q, c] += h
            pm[q, c] -= h
            Lp, ip = loss(pp)
            Lm, im = loss(pm)
            if not (np.array_equal(ip, idx) and np.array_equal(im, idx)):
                continue
            assert grad[q, c] == pytest.approx((Lp - Lm) / (2 * h), rel=1e-6, abs=1e-7)
            tested += 1
    assert tested >= 30


@pytest.mark.parametrize("name", ["points_small", "points_soup"])
def test_point_band_oracle_equals_whole_oracle(name):
    """The band reduction the dense full-size GPU check uses
    (parity.point_oracle_band: the oracle on one image's points near a band
    of 16 rows, indices mapped back) gives exactly the whole-batch oracle on
    every pixel of every image."""
    from parity import point_oracle_band

    w = make_point_workload(name)
    pts = np.asarray(w.points, np.float32).reshape(-1, 3)
    full = rasterize_points(w.points, w.offsets, w.H, w.W, w.K, w.radius)
    for n in range(len(w.offsets) - 1):
        for r0 in range(0, w.H, 16):
            r1 = min(w.H, r0 + 16)
            band = point_oracle_band(rasterize_points, w, n, r0, r1, pts)
            for a, b in zip(band, full):
                np.testing.assert_array_equal(a, b[n].reshape(w.H * w.W, w.K)[r0 * w.W:r1 * w.W])

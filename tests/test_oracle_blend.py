"""Pins of the second-stage (blend) oracle: hand-worked single- and two-face
values, the empty pixel, limits, slot-order and padding invariance, and
central finite differences of its backward pass."""

import math

import numpy as np
import pytest

from oracle.blend import BlendParams, blend_backward, blend_forward


def _one_pixel(faces, z, d, K=4):
    p2f = np.full((1, K), -1, np.int64)
    zb = np.full((1, K), -1.0)
    ds = np.full((1, K), -1.0)
    for k, (f, zz, dd) in enumerate(zip(faces, z, d)):
        p2f[0, k], zb[0, k], ds[0, k] = f, zz, dd
    return p2f, zb, ds


COLORS = np.array([[0.1, 0.2, 0.3], [0.9, 0.5, 0.1], [0.25, 0.75, 0.5], [0.0, 1.0, 0.0]])


def test_single_face_far_background():
    # sigma = 1e-4, d = -0.5e-4: p = 1 / (1 + e^-0.5); the background weight
    # exp((eps - 98/99) / 1e-4) underflows to 0, so rgb is the face colour
    prm = BlendParams()
    p2f, zb, ds = _one_pixel([2], [2.0], [-0.5e-4])
    out = blend_forward(p2f, zb, ds, COLORS, prm)[0]
    p = 1.0 / (1.0 + math.exp(-0.5))
    assert out[3] == pytest.approx(0.6224593312018546, abs=1e-15)
    assert out[3] == pytest.approx(p, abs=1e-15)
    np.testing.assert_allclose(out[:3], COLORS[2], atol=1e-15)


def test_single_face_near_background():
    # zfar = 3, z = 2.9: zeta = 0.1 / 2 = 0.05, background weight
    # exp((1e-10 - 0.05) / 0.1) = exp(-0.5 + 1e-9); d = 0: p = 1/2
    prm = BlendParams(sigma=1e-3, gamma=0.1, znear=1.0, zfar=3.0, background=(0.0, 0.0, 1.0))
    p2f, zb, ds = _one_pixel([1], [2.9], [0.0])
    out = blend_forward(p2f, zb, ds, COLORS, prm)[0]
    bw = math.exp(-0.5 + 1e-9)
    want = (0.5 * COLORS[1] + bw * np.array([0.0, 0.0, 1.0])) / (0.5 + bw)
    np.testing.assert_allclose(out[:3], want, rtol=1e-13)
    assert out[3] == pytest.approx(0.5, abs=1e-15)


def test_two_faces_same_depth():
    prm = BlendParams(sigma=2e-4)
    p2f, zb, ds = _one_pixel([0, 3], [1.5, 1.5], [-1e-4, 3e-4])
    out = blend_forward(p2f, zb, ds, COLORS, prm)[0]
    p1 = 1 / (1 + math.exp(-0.5))
    p2 = 1 / (1 + math.exp(1.5))
    np.testing.assert_allclose(out[:3], (p1 * COLORS[0] + p2 * COLORS[3]) / (p1 + p2), rtol=1e-13)
    assert out[3] == pytest.approx(1 - (1 - p1) * (1 - p2), abs=1e-15)


def test_empty_pixel_is_background():
    prm = BlendParams(background=(0.3, 0.2, 0.1))
    p2f, zb, ds = _one_pixel([], [], [])
    out = blend_forward(p2f, zb, ds, COLORS, prm)[0]
    np.testing.assert_array_equal(out, [0.3, 0.2, 0.1, 0.0])
    gz, gd = blend_backward(p2f, zb, ds, COLORS, prm, np.ones((1, 4)))
    assert not gz.any() and not gd.any()


def test_nearer_face_dominates_for_small_gamma():
    prm = BlendParams(gamma=1e-6)
    p2f, zb, ds = _one_pixel([0, 1], [1.2, 1.3], [-1e-4, -1e-4])
    out = blend_forward(p2f, zb, ds, COLORS, prm)[0]
    np.testing.assert_allclose(out[:3], COLORS[0], atol=1e-12)


def _random_case(seed, P=50, K=5):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, K + 1, P)
    p2f = np.full((P, K), -1, np.int64)
    zb = np.full((P, K), -1.0)
    ds = np.full((P, K), -1.0)
    for i in range(P):
        p2f[i, :n[i]] = rng.integers(0, len(COLORS), n[i])
        zb[i, :n[i]] = np.sort(rng.uniform(1.0, 3.0, n[i]))
        ds[i, :n[i]] = rng.normal(0, 2e-4, n[i])
    return p2f, zb, ds


def test_slot_order_and_padding_do_not_matter():
    prm = BlendParams(gamma=1e-2, zfar=5.0)
    p2f, zb, ds = _random_case(1)
    ref = blend_forward(p2f, zb, ds, COLORS, prm)
    perm = np.random.default_rng(2).permutation(p2f.shape[1])
    np.testing.assert_allclose(blend_forward(p2f[:, perm], zb[:, perm], ds[:, perm], COLORS, prm), ref, rtol=1e-12)
    zb2, ds2 = zb.copy(), ds.copy()
    pad = p2f < 0
    zb2[pad] = 7.0
    ds2[pad] = -3.0
    np.testing.assert_array_equal(blend_forward(p2f, zb2, ds2, COLORS, prm), ref)


def test_outputs_are_convex_combinations():
    prm = BlendParams(gamma=1e-2, zfar=5.0, background=(0.5, 0.5, 0.5))
    p2f, zb, ds = _random_case(3, P=200)
    out = blend_forward(p2f, zb, ds, COLORS, prm)
    assert (out[:, 3] >= 0).all() and (out[:, 3] <= 1).all()
    lo = np.minimum(COLORS.min(0), 0.5)
    hi = np.maximum(COLORS.max(0), 0.5)
    assert (out[:, :3] >= lo - 1e-12).all() and (out[:, :3] <= hi + 1e-12).all()


@pytest.mark.parametrize("seed", [4, 5])
def test_backward_matches_finite_differences(seed):
    prm = BlendParams(sigma=2e-4, gamma=2e-2, zfar=5.0, background=(0.2, 0.9, 0.4))
    p2f, zb, ds = _random_case(seed, P=30)
    g = np.random.default_rng(seed + 10).normal(size=(30, 4))
    gz, gd = blend_backward(p2f, zb, ds, COLORS, prm, g)

    def loss(z, d):
        return float((blend_forward(p2f, z, d, COLORS, prm) * g).sum())

    hz, hd = 1e-7, 1e-9
    for i in range(30):
        for k in range(p2f.shape[1]):
            if p2f[i, k] < 0:
                assert gz[i, k] == 0 and gd[i, k] == 0
                continue
            z1, z2 = zb.copy(), zb.copy()
            z1[i, k] += hz
            z2[i, k] -= hz
            fz = (loss(z1, ds) - loss(z2, ds)) / (2 * hz)
            d1, d2 = ds.copy(), ds.copy()
            d1[i, k] += hd
            d2[i, k] -= hd
            fd = (loss(zb, d1) - loss(zb, d2)) / (2 * hd)
            assert gz[i, k] == pytest.approx(fz, rel=1e-5, abs=1e-6)
            assert gd[i, k] == pytest.approx(fd, rel=1e-5, abs=1e-3)

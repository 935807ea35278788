"""Pins of the second-stage (blend) oracle: hand-worked single- and two-face
values (forward, backward and the per-slot error scale), a very sharp sigma
whose weights all underflow binary64, the empty pixel, limits, slot-order
and padding invariance, and central finite differences of its backward
pass. test_oracle_blend_mutants.py runs the same pins against planted
mistakes."""

import math

import numpy as np
import pytest

from oracle.blend import BlendParams, blend_backward, blend_backward_scale, blend_forward


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


# ---------------------------------------------------------------------------
# hand-worked backward values and per-slot error scales
# ---------------------------------------------------------------------------

def test_scale_one_face_hand_worked():
    # One face, d = 0: p = q = 1/2. znear 1, zfar 3, z = 2: zeta = 1/2 =
    # zeta_max, so the face weight is p = 1/2 and the background weight
    # exp((0 - 1/2) / (1/2)) = 1/e. Normalised: face e/(e+2), background
    # 2/(e+2). The background colour equals the face colour c, so rgb = c.
    #   colour terms per channel: |g_c| (|c_c| + |rgb_c|) = 2 |g_c| c_c;
    #   with c = (1/4, 1/2, 1), g = (1, -2, 1/2): S = 2 (1/4 + 1 + 1/2) = 7/2
    #   grad_zbuf scale  S * e/(e+2) / ((zfar - znear) gamma) = (7/2) e/(e+2)
    #   grad_dists scale S * e/(e+2) * q / sigma + |g_a| (1 - alpha) p / sigma
    #                  = (7/2) e/(e+2) * 2 + 3 * (1/4) * 4 = 7e/(e+2) + 3
    # The colour terms cancel exactly (c - rgb = 0): grad_zbuf = 0 and
    # grad_dists = -g_a (1 - alpha) p / sigma = -3.
    prm = BlendParams(sigma=0.25, gamma=0.5, znear=1.0, zfar=3.0, eps=0.0, background=(0.25, 0.5, 1.0))
    colors = np.array([[0.25, 0.5, 1.0]])
    p2f, zb, ds = _one_pixel([0], [2.0], [0.0], K=2)
    g = np.array([[1.0, -2.0, 0.5, 3.0]])
    e = math.e
    sz, sd = blend_backward_scale(p2f, zb, ds, colors, prm, g)
    assert sz[0, 0] == pytest.approx(3.5 * e / (e + 2), rel=1e-14)
    assert sd[0, 0] == pytest.approx(7 * e / (e + 2) + 3, rel=1e-14)
    assert sz[0, 1] == 0 and sd[0, 1] == 0
    gz, gd = blend_backward(p2f, zb, ds, colors, prm, g)
    assert abs(gz[0, 0]) <= 1e-14
    assert gd[0, 0] == pytest.approx(-3.0, rel=1e-14)
    out = blend_forward(p2f, zb, ds, colors, prm)[0]
    np.testing.assert_allclose(out, [0.25, 0.5, 1.0, 0.5], rtol=1e-14)


def test_scale_two_faces_hand_worked():
    # Two faces at one depth (zeta equal), d1 = 0 and d2 = sigma ln 3:
    # p1 = 1/2, q1 = 1/2, p2 = 1/4, q2 = 3/4. gamma = 1e-3: the background
    # weight exp(-500) is negligible against them, so the normalised weights
    # are 2/3 and 1/3. Colours red and green: rgb = (2/3, 1/3, 0).
    # g = (1, 1, 1, 2):
    #   g . (c1 - rgb) = 1/3 - 1/3 = 0 and g . (c2 - rgb) = -2/3 + 2/3 = 0, so
    #   the colour gradients vanish; their scales S_k = sum_c |g_c| (|c_kc| +
    #   |rgb_c|) are S1 = (1 + 2/3) + 1/3 = 2 and S2 = 2/3 + (1 + 1/3) = 2.
    #   1 - alpha = q1 q2 = 3/8; sigma = 1/2; (zfar - znear) gamma = 2e-3.
    #   grad_zbuf scales: 2 * (2/3) / 2e-3 = 2000/3, 2 * (1/3) / 2e-3 = 1000/3
    #   grad_dists scales: S_k what_k q_k / sigma + |g_a| (3/8) p_k / sigma
    #     k=1: 2 (2/3)(1/2) 2 + 2 (3/8)(1/2) 2 = 4/3 + 3/4 = 25/12
    #     k=2: 2 (1/3)(3/4) 2 + 2 (3/8)(1/4) 2 = 1 + 3/8 = 11/8
    #   grad_dists = -g_a (1 - alpha) p_k / sigma = -3/4 and -3/8.
    sigma = 0.5
    prm = BlendParams(sigma=sigma, gamma=1e-3, znear=1.0, zfar=3.0, eps=0.0, background=(0.0, 0.0, 1.0))
    colors = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    p2f, zb, ds = _one_pixel([0, 1], [2.0, 2.0], [0.0, sigma * math.log(3.0)], K=3)
    g = np.array([[1.0, 1.0, 1.0, 2.0]])
    sz, sd = blend_backward_scale(p2f, zb, ds, colors, prm, g)
    np.testing.assert_allclose(sz[0, :2], [2000 / 3, 1000 / 3], rtol=1e-13)
    np.testing.assert_allclose(sd[0, :2], [25 / 12, 11 / 8], rtol=1e-13)
    assert sz[0, 2] == 0 and sd[0, 2] == 0
    gz, gd = blend_backward(p2f, zb, ds, colors, prm, g)
    np.testing.assert_allclose(gz[0, :2], 0.0, atol=1e-10)
    np.testing.assert_allclose(gd[0, :2], [-0.75, -0.375], rtol=1e-13)
    out = blend_forward(p2f, zb, ds, colors, prm)[0]
    np.testing.assert_allclose(out, [2 / 3, 1 / 3, 0.0, 5 / 8], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("seed", [6, 7])
def test_scale_bounds_every_gradient(seed):
    # each gradient is a signed sum of the terms whose magnitudes the scale
    # adds up, so |gradient| <= scale everywhere (with rounding slack)
    prm = BlendParams(sigma=2e-4, gamma=2e-2, zfar=5.0, background=(0.2, 0.9, 0.4))
    p2f, zb, ds = _random_case(seed, P=200)
    g = np.random.default_rng(seed).normal(size=(200, 4))
    gz, gd = blend_backward(p2f, zb, ds, COLORS, prm, g)
    sz, sd = blend_backward_scale(p2f, zb, ds, COLORS, prm, g)
    assert (np.abs(gz) <= sz * (1 + 1e-12)).all()
    assert (np.abs(gd) <= sd * (1 + 1e-12)).all()
    assert ((sz > 0) == (p2f >= 0)).all() and ((sd > 0) == (p2f >= 0)).all()


def test_binary32_evaluation_within_scale():
    # what the scale is for: the same sums evaluated in binary32 differ from
    # binary64 by a small multiple of the unit roundoff times the scale,
    # including where the terms cancel exactly (a single face whose colour
    # equals the blended colour)
    prm = BlendParams(sigma=2e-4, gamma=2e-2, zfar=5.0, background=(0.2, 0.9, 0.4))
    p2f, zb, ds = _random_case(8, P=300)
    g = np.random.default_rng(9).normal(size=(300, 4))
    gz, gd = blend_backward(p2f, zb, ds, COLORS, prm, g)
    sz, sd = blend_backward_scale(p2f, zb, ds, COLORS, prm, g)
    f = np.float32
    gz32, gd32 = blend_backward(p2f, zb.astype(f).astype(np.float64), ds.astype(f).astype(np.float64),
                                COLORS.astype(f).astype(np.float64), prm, g.astype(f).astype(np.float64))
    # rounding the inputs to binary32 moves each term by a few units of 2^-24
    # times its size (the weight exponents amplify depth rounding by
    # |z| / ((zfar - znear) gamma) ~ 50)
    u = 2.0 ** -24
    assert (np.abs(gz32 - gz) <= 200 * u * sz + 1e-300).all()
    assert (np.abs(gd32 - gd) <= 200 * u * sd + 1e-300).all()


# ---------------------------------------------------------------------------
# a sigma far below the squared distances: every weight underflows binary64
# ---------------------------------------------------------------------------

def test_very_sharp_sigma_keeps_the_weight_ratio():
    # d1 / sigma = 2000 and d2 / sigma = 2001 (both faces outside), one depth:
    # p_k = 1 / (1 + e^(d_k/sigma)) are e^-2000 and e^-2001 to relative
    # e^-2000, far below the smallest binary64 number, but their ratio is e.
    # gamma = 1e-4, zeta = 1/2, eps = 0: the background weight e^-5000 is
    # smaller still (relative e^-3000). So rgb = (e c1 + c2) / (e + 1), and
    # alpha = 1 - (1 - p1)(1 - p2) ~ e^-2000 rounds to 0.
    # With g = (1, 0, 0, 0), c1 red, c2 green: rgb_r = e/(e+1),
    # g . (c1 - rgb) = 1/(e+1), g . (c2 - rgb) = -e/(e+1); q_k = 1, so
    # grad_dists_k = -(g . (c_k - rgb)) what_k / sigma = -/+ e / ((e+1)^2 sigma)
    # and grad_zbuf_k = the same with (zfar - znear) gamma = 2e-4 for sigma.
    sigma = 3e-7
    prm = BlendParams(sigma=sigma, gamma=1e-4, znear=1.0, zfar=3.0, eps=0.0, background=(0.0, 0.0, 1.0))
    colors = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    p2f, zb, ds = _one_pixel([0, 1], [2.0, 2.0], [2000 * sigma, 2001 * sigma], K=2)
    e = math.e
    out = blend_forward(p2f, zb, ds, colors, prm)[0]
    np.testing.assert_allclose(out, [e / (e + 1), 1 / (e + 1), 0.0, 0.0], rtol=1e-10, atol=1e-300)
    gz, gd = blend_backward(p2f, zb, ds, colors, prm, np.array([[1.0, 0.0, 0.0, 0.0]]))
    k = e / (e + 1) ** 2
    np.testing.assert_allclose(gd[0], [-k / sigma, k / sigma], rtol=1e-9)
    np.testing.assert_allclose(gz[0], [-k / 2e-4, k / 2e-4], rtol=1e-9)
    sz, sd = blend_backward_scale(p2f, zb, ds, colors, prm, np.array([[1.0, 0.0, 0.0, 0.0]]))
    assert np.isfinite(sz).all() and np.isfinite(sd).all() and (sd > 0).all()

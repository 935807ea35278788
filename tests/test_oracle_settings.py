"""Pins of the oracle's rasterizer settings: perspective-correct barycentrics,
back-face culling and unclipped barycentrics (rocketrecap summary, "32:56
Technical Bug Fix", names the perspective_correct setting; the readings are
in oracle/raster_oracle_impl.h).

- a hand-worked perspective case with exact screen-space barycentrics;
- perspective results against the reciprocal form of the same interpolation
  (1/z linear in screen space), formed here from the oracle's own
  screen-space output;
- culling against the unculled oracle on a face list whose back faces were
  made degenerate, and the first-hit identity on closed outward meshes;
- unclipped barycentrics reproduce the pixel centre as an affine combination
  of the vertices, and match the perspective reciprocal form;
- central finite differences of the backward pass under every setting.
"""

import numpy as np
import pytest

from oracle import CULL_BACKFACES, PERSPECTIVE, UNCLIPPED_BARY
from workloads import icosphere

H = W = 16
STEP = 1e-6


def _hand_case():
    # pixel (1, 1) of a 4x4 image has its centre at (-0.25, -0.25), which is
    # 0.5 v0 + 0.25 v1 + 0.25 v2 exactly
    v = np.array([[-0.5, -0.5, 1.0], [0.5, -0.5, 2.0], [-0.5, 0.5, 4.0]])
    return v, np.array([[0, 1, 2]], np.int64), np.array([0, 1], np.int64)


@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_perspective_hand_case(oracle_mod, precision):
    v, f, o = _hand_case()
    _, zb, ba, _ = oracle_mod.rasterize(v, f, o, 4, 4, 1, 0.0, precision=precision)
    # screen space: b = (1/2, 1/4, 1/4), z = 1/2 + 2/4 + 4/4
    assert zb[0, 1, 1, 0] == 2.0
    np.testing.assert_array_equal(ba[0, 1, 1, 0], [0.5, 0.25, 0.25])
    p2f, zb, ba, _ = oracle_mod.rasterize(v, f, o, 4, 4, 1, 0.0, precision=precision, settings=PERSPECTIVE)
    # weights b_k / z_k = (1/2, 1/8, 1/16), sum 11/16: bary (8, 2, 1) / 11, z = 16/11
    tol = 4e-7 if precision == "f32" else 1e-15
    assert p2f[0, 1, 1, 0] == 0
    assert zb[0, 1, 1, 0] == pytest.approx(16 / 11, rel=tol)
    np.testing.assert_allclose(ba[0, 1, 1, 0], np.array([8, 2, 1]) / 11, rtol=tol)


def _scene(seed, nmesh=2, nf=6, zlo=0.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    verts, faces, offsets = [], [], [0]
    for _ in range(nmesh):
        for _ in range(nf):
            c = rng.uniform(-0.6, 0.6, (1, 2))
            xy = c + rng.normal(0.0, 0.35, (3, 2))
            z = rng.uniform(zlo, 3.0) + rng.normal(0.0, 0.3, (3, 1))
            z = np.maximum(z, zlo / 2)
            faces.append(np.arange(len(verts), len(verts) + 3))
            verts.extend(np.concatenate([xy, z], axis=1))
        offsets.append(offsets[-1] + nf)
    return np.asarray(verts), np.asarray(faces, np.int64), np.asarray(offsets, np.int64)


def _slots(p2f):
    return np.argwhere(p2f >= 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_perspective_matches_reciprocal_form(oracle_mod, seed):
    v, f, o = _scene(seed)
    K, blur = 12, 0.01
    screen = oracle_mod.rasterize(v, f, o, H, W, K, blur, precision="f64")
    persp = oracle_mod.rasterize(v, f, o, H, W, K, blur, precision="f64", settings=PERSPECTIVE)
    # same candidate sets (inclusion does not depend on the setting); K holds them all
    assert (screen[0][..., -1] < 0).all()
    np.testing.assert_array_equal(np.sort(screen[0], axis=-1), np.sort(persp[0], axis=-1))
    checked = 0
    for idx in _slots(persp[0]):
        n, i, j, k = idx
        face = persp[0][n, i, j, k]
        ks = int(np.nonzero(screen[0][n, i, j] == face)[0][0])
        c = screen[2][n, i, j, ks]              # clipped, renormalised screen weights
        z = v[f[face], 2]
        inv = c / z
        zp = 1.0 / inv.sum()
        assert persp[1][n, i, j, k] == pytest.approx(zp, rel=1e-12)
        np.testing.assert_allclose(persp[2][n, i, j, k], inv * zp, rtol=1e-12, atol=1e-15)
        assert persp[3][n, i, j, k] == screen[3][n, i, j, ks]
        checked += 1
    assert checked > 50
    # the lists are ordered by the perspective depth
    z = np.where(persp[0] >= 0, persp[1], 1e300)
    assert (np.diff(z, axis=-1) >= 0).all()


def test_perspective_skips_faces_behind_the_camera(oracle_mod):
    v, f, o = _hand_case()
    v = v.copy()
    v[2, 2] = -0.5                          # one vertex behind the camera
    screen = oracle_mod.rasterize(v, f, o, 4, 4, 1, 0.0)
    persp = oracle_mod.rasterize(v, f, o, 4, 4, 1, 0.0, settings=PERSPECTIVE)
    assert (screen[0] == 0).any()
    assert (persp[0] == -1).all()


@pytest.mark.parametrize("seed", [3, 4])
def test_culling_equals_degenerate_back_faces(oracle_mod, seed):
    v, f, o = _scene(seed, nf=10)
    p = v[f]
    A = (p[:, 1, 0] - p[:, 0, 0]) * (p[:, 2, 1] - p[:, 0, 1]) - (p[:, 1, 1] - p[:, 0, 1]) * (p[:, 2, 0] - p[:, 0, 0])
    assert (np.abs(A) > 1e-3).all() and (A > 0).any() and (A < 0).any()
    f_front = f.copy()
    f_front[A > 0] = f[A > 0][:, :1]        # all three indices equal: A == 0, never a candidate
    for settings in (0, PERSPECTIVE, UNCLIPPED_BARY):
        culled = oracle_mod.rasterize(v, f, o, H, W, 4, 0.01, settings=settings | CULL_BACKFACES)
        ref = oracle_mod.rasterize(v, f_front, o, H, W, 4, 0.01, settings=settings)
        for a, b in zip(culled, ref):
            np.testing.assert_array_equal(a, b)


def test_culling_keeps_the_first_hit_of_closed_meshes(oracle_mod):
    # outward-oriented icospheres: every pixel's nearest face is front-facing
    rng = np.random.Generator(np.random.PCG64(7))
    verts, faces, offsets = [], [], [0]
    for n in range(2):
        sv, sf = icosphere(2)
        q = rng.normal(size=4)
        q /= np.linalg.norm(q)
        a, b, c, d = q
        Rm = np.array([[a*a+b*b-c*c-d*d, 2*(b*c-a*d), 2*(b*d+a*c)],
                       [2*(b*c+a*d), a*a-b*b+c*c-d*d, 2*(c*d-a*b)],
                       [2*(b*d-a*c), 2*(c*d+a*b), a*a-b*b-c*c+d*d]])
        sv = sv @ Rm.T * 0.7 + np.array([0.05 * n, -0.03, 2.0])
        faces.append(sf + len(verts) if verts else sf)
        verts.extend(sv)
        offsets.append(offsets[-1] + len(sf))
    v = np.asarray(verts)
    f = np.concatenate(faces)
    o = np.asarray(offsets, np.int64)
    full = oracle_mod.rasterize(v, f, o, 32, 32, 1, 0.0)
    culled = oracle_mod.rasterize(v, f, o, 32, 32, 1, 0.0, settings=CULL_BACKFACES)
    assert (full[0] >= 0).mean() > 0.3
    for a, b in zip(full, culled):
        np.testing.assert_array_equal(a, b)
    # and with K = 2 the culled second slot is empty wherever the sphere is hit once from the front
    full2 = oracle_mod.rasterize(v, f, o, 32, 32, 2, 0.0)
    culled2 = oracle_mod.rasterize(v, f, o, 32, 32, 2, 0.0, settings=CULL_BACKFACES)
    assert (full2[0][..., 1] >= 0).sum() > 0.9 * (full2[0][..., 0] >= 0).sum()
    assert (culled2[0][..., 1] < 0).all()


@pytest.mark.parametrize("seed", [5, 6])
def test_unclipped_barycentrics(oracle_mod, seed):
    v, f, o = _scene(seed)
    K, blur = 12, 0.02
    clipped = oracle_mod.rasterize(v, f, o, H, W, K, blur, precision="f64")
    raw = oracle_mod.rasterize(v, f, o, H, W, K, blur, precision="f64", settings=UNCLIPPED_BARY)
    for a, b in ((clipped[0], raw[0]), (clipped[1], raw[1]), (clipped[3], raw[3])):
        np.testing.assert_array_equal(a, b)
    rawp = oracle_mod.rasterize(v, f, o, H, W, K, blur, precision="f64", settings=UNCLIPPED_BARY | PERSPECTIVE)
    persp = oracle_mod.rasterize(v, f, o, H, W, K, blur, precision="f64", settings=PERSPECTIVE)
    for a, b in ((persp[0], rawp[0]), (persp[1], rawp[1]), (persp[3], rawp[3])):
        np.testing.assert_array_equal(a, b)
    outside = 0
    for n, i, j, k in _slots(raw[0]):
        face = raw[0][n, i, j, k]
        P = v[f[face]]
        b = raw[2][n, i, j, k]
        px, py = (2 * j + 1) / W - 1, (2 * i + 1) / H - 1
        # an affine combination of the vertices that lands on the pixel centre
        assert b.sum() == pytest.approx(1.0, abs=1e-12)
        np.testing.assert_allclose(b @ P[:, :2], [px, py], atol=1e-12)
        outside += bool((b < 0).any())
        if (b > 0).all() and (b < 1).all():
            np.testing.assert_allclose(b, clipped[2][n, i, j, k], rtol=1e-12)
        # perspective form of the same unclipped weights
        kp = int(np.nonzero(rawp[0][n, i, j] == face)[0][0])
        w = b / P[:, 2]
        np.testing.assert_allclose(rawp[2][n, i, j, kp], w / w.sum(), rtol=1e-9, atol=1e-12)
    assert outside > 10


def _fd_scene(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    nf = int(rng.integers(1, 5))
    K = int(rng.integers(1, 4))
    blur = float(rng.choice([0.0, 1e-3, 1e-2]))
    c = rng.uniform(-0.6, 0.6, (nf, 1, 2))
    xy = c + rng.normal(0.0, 0.35, (nf, 3, 2))
    z = rng.uniform(1.0, 3.0, (nf, 1, 1)) + rng.normal(0.0, 0.3, (nf, 3, 1))
    v = np.concatenate([xy, z], axis=2).reshape(-1, 3)
    faces = np.arange(3 * nf, dtype=np.int64).reshape(nf, 3)
    g = {
        "zbuf": rng.standard_normal((1, H, W, K)),
        "bary": rng.standard_normal((1, H, W, K, 3)),
        "dists": rng.standard_normal((1, H, W, K)) * 10,
    }
    return v, faces, np.array([0, nf], np.int64), K, blur, g


def _loss(oracle, v, f, o, K, blur, g, settings):
    p2f, zb, ba, di, st = oracle.rasterize(v, f, o, H, W, K, blur, precision="f64", with_state=True,
                                           settings=settings)
    return (g["zbuf"] * zb).sum() + (g["bary"] * ba).sum() + (g["dists"] * di).sum(), p2f, st


SETTINGS = {"persp": PERSPECTIVE, "raw": UNCLIPPED_BARY, "raw_persp": UNCLIPPED_BARY | PERSPECTIVE,
            "cull_persp": CULL_BACKFACES | PERSPECTIVE}


@pytest.mark.parametrize("seed", list(range(4)))
@pytest.mark.parametrize("name", list(SETTINGS))
def test_backward_matches_finite_differences(oracle_mod, name, seed):
    settings = SETTINGS[name]
    v, f, o, K, blur, g = _fd_scene(seed)
    _, p2f, st = _loss(oracle_mod, v, f, o, K, blur, g, settings)
    grad = oracle_mod.backward(v, f, o, H, W, K, blur, p2f, g["zbuf"].astype(np.float32),
                               g["bary"].astype(np.float32), g["dists"].astype(np.float32),
                               precision="f64", settings=settings)
    g32 = {k: a.astype(np.float32).astype(np.float64) for k, a in g.items()}
    tested = skipped = 0
    for vi in np.unique(f):
        for c in range(3):
            vp, vm = v.copy(), v.copy()
            vp[vi, c] += STEP
            vm[vi, c] -= STEP
            Lp, pp, sp = _loss(oracle_mod, vp, f, o, K, blur, g32, settings)
            Lm, pm, sm = _loss(oracle_mod, vm, f, o, K, blur, g32, settings)
            if not (np.array_equal(pp, p2f) and np.array_equal(pm, p2f)
                    and np.array_equal(sp, st) and np.array_equal(sm, st)):
                skipped += 1
                continue
            fd = (Lp - Lm) / (2 * STEP)
            an = grad[vi, c]
            assert abs(fd - an) <= 1e-5 * (1 + abs(an)), (vi, c, fd, an)
            tested += 1
    assert tested >= 0.85 * (tested + skipped), (tested, skipped)
    if (p2f >= 0).any():
        assert np.abs(grad).max() > 0

"""Pins of the projection oracle (oracle/project.py): hand-worked pinhole
cases, the identity camera, invariance of x and y to a scale of the camera,
the workload construction (projection gives back the screen-space
vertices), and central finite differences of its backward pass."""

import numpy as np
import pytest

from oracle.project import (project_backward, project_backward_error_bound, project_forward,
                            project_forward_error_bound)
from workloads import make_workload, projection_inputs


def _pinhole(f, t=(0.0, 0.0, 0.0)):
    M = np.zeros((4, 4))
    M[0, 0] = M[1, 1] = f
    M[2, 2] = M[3, 2] = 1.0
    M[0, 3], M[1, 3] = f * t[0], f * t[1]
    M[2, 3] = M[3, 3] = t[2]
    return M


def test_pinhole_hand_case():
    # f = 2: (1, -0.5, 4) -> (2 * 1 / 4, 2 * -0.5 / 4, 4); on the axis -> (0, 0, z)
    X = np.array([[1.0, -0.5, 4.0], [0.0, 0.0, 2.5]])
    out = project_forward(X, [0, 2], _pinhole(2.0)[None])
    np.testing.assert_array_equal(out, [[0.5, -0.25, 4.0], [0.0, 0.0, 2.5]])
    # a translation along the axis moves the depth: (1, 1, 1) + (0, 0, 1) -> (1, 1, 2) / 2 * 2
    out = project_forward(np.array([[1.0, 1.0, 1.0]]), [0, 1], _pinhole(2.0, (0.0, 0.0, 1.0))[None])
    np.testing.assert_array_equal(out, [[1.0, 1.0, 2.0]])


def test_identity_camera_and_heterogeneous_batch():
    rng = np.random.default_rng(0)
    X = rng.normal(size=(7, 3))
    eye = np.eye(4)
    out = project_forward(X, [0, 3, 3, 7], np.stack([eye, 2 * eye, eye]))
    np.testing.assert_allclose(out[:3], X[:3], rtol=0, atol=0)
    # mesh 1 is empty; mesh 2 takes vertices 3..6 with the identity
    np.testing.assert_allclose(out[3:], X[3:], rtol=0, atol=0)


def test_scaled_camera_keeps_xy():
    rng = np.random.default_rng(1)
    X = rng.normal(size=(20, 3))
    M = rng.normal(size=(1, 4, 4))
    M[0, 3] = [0.1, 0.2, 0.3, 5.0]
    a = project_forward(X, [0, 20], M)
    b = project_forward(X, [0, 20], 3.0 * M)
    np.testing.assert_allclose(b[:, :2], a[:, :2], rtol=1e-13)
    np.testing.assert_allclose(b[:, 2], 3.0 * a[:, 2], rtol=1e-13)


@pytest.mark.parametrize("name", ["small_hetero", "spheres8_137"])
def test_workload_cameras_give_back_the_screen_vertices(name):
    w = make_workload(name)
    X, vo, M = projection_inputs(w)
    out = project_forward(X, vo, M)
    np.testing.assert_allclose(out, w.verts, atol=2e-6, rtol=0)
    b = project_forward_error_bound(X, vo, M)
    assert (b > 0).all() and (b < 1e-5).all()


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(2)
    X = rng.normal(size=(9, 3))
    X[:, 2] += 4.0
    vo = [0, 4, 9]
    M = np.stack([_pinhole(1.7, (0.1, -0.2, 0.5)), _pinhole(2.2)]) + rng.normal(0, 0.05, (2, 4, 4))
    g = rng.normal(size=(9, 3))
    gX, gM = project_backward(X, vo, M, g)

    def loss(XX, MM):
        return float((project_forward(XX, vo, MM) * g).sum())

    h = 1e-6
    for i in range(9):
        for c in range(3):
            Xp, Xm = X.copy(), X.copy()
            Xp[i, c] += h
            Xm[i, c] -= h
            assert gX[i, c] == pytest.approx((loss(Xp, M) - loss(Xm, M)) / (2 * h), rel=1e-6, abs=1e-8)
    for n in range(2):
        for r in range(4):
            for c in range(4):
                Mp, Mm = M.copy(), M.copy()
                Mp[n, r, c] += h
                Mm[n, r, c] -= h
                assert gM[n, r, c] == pytest.approx((loss(X, Mp) - loss(X, Mm)) / (2 * h), rel=1e-6, abs=1e-8)


def test_error_bound_holds_for_float32_evaluation():
    # the bound covers a plain binary32 evaluation in the stated order
    w = make_workload("small_hetero")
    X, vo, M = projection_inputs(w)
    ref = project_forward(X, vo, M)
    bound = project_forward_error_bound(X, vo, M)
    mesh = np.repeat(np.arange(len(vo) - 1), np.diff(vo))
    Mm = M[mesh]
    f = np.float32
    h = [(((Mm[:, r, 0] * X[:, 0]).astype(f) + (Mm[:, r, 1] * X[:, 1]).astype(f)).astype(f)
          + (Mm[:, r, 2] * X[:, 2]).astype(f)).astype(f) + Mm[:, r, 3] for r in range(4)]
    h = [a.astype(f) for a in h]
    out32 = np.stack([(h[0] / h[3]).astype(f), (h[1] / h[3]).astype(f), h[2]], axis=1)
    assert (np.abs(out32 - ref) <= bound).all()


def test_backward_error_bound_holds_for_float32_evaluation():
    w = make_workload("small_hetero")
    X, vo, M = projection_inputs(w)
    g = np.random.default_rng(4).standard_normal((w.V, 3)).astype(np.float32)
    f = np.float32
    mesh = np.repeat(np.arange(len(vo) - 1), np.diff(vo))
    Mm = M[mesh]
    h = [((((Mm[:, r, 0] * X[:, 0]) + (Mm[:, r, 1] * X[:, 1])) + (Mm[:, r, 2] * X[:, 2])) + Mm[:, r, 3]).astype(f)
         for r in range(4)]
    px, py = h[0] / h[3], h[1] / h[3]
    gh = [g[:, 0] / h[3], g[:, 1] / h[3], g[:, 2], -((g[:, 0] * px) + (g[:, 1] * py)) / h[3]]
    gv = np.stack([(((Mm[:, 0, c] * gh[0]) + (Mm[:, 1, c] * gh[1])) + (Mm[:, 2, c] * gh[2])) + (Mm[:, 3, c] * gh[3])
                   for c in range(3)], axis=1)
    assert gv.dtype == np.float32
    rgx, rgm = project_backward(X, vo, M, g)
    bv, bm = project_backward_error_bound(X, vo, M, g, cam_sum_depth=np.diff(vo) // 256 + 10)
    assert (np.abs(gv - rgx) <= bv).all()
    # camera entries summed in float32, 256 terms at a time (numpy's pairwise
    # sum within each, depth <= 8), the partial sums one after the other
    Xh = np.concatenate([X, np.ones((len(X), 1), f)], axis=1)
    gm = np.stack(gh, axis=1)[:, :, None] * Xh[:, None, :]
    gc = np.zeros(M.shape, f)
    for n in range(len(vo) - 1):
        for b0 in range(vo[n], vo[n + 1], 256):
            gc[n] += gm[b0:min(b0 + 256, vo[n + 1])].sum(0, dtype=f)
    assert (np.abs(gc - rgm) <= bm + 1e-30).all()
    # and it is not vacuous: a relative error of 1e-4 on one entry breaks it
    assert not (np.abs(gv * (1 + 1e-4) - rgx) <= bv).all()


def test_error_bounds_hand_cases():
    # The bounds written out by hand for one vertex X = (1, 1, 1), with
    # u = 2^-24 and g4 = 4u / (1 - 4u) (four rounded products summed).
    u = 2.0 ** -24
    g4 = 4 * u / (1 - 4 * u)
    X = np.array([[1.0, 1.0, 1.0]])
    # identity camera: h = (1, 1, 1, 1), every |M||X| row sum is 1, so each
    # h_r is off by g4; x = h0 / h3 takes both operands' errors and one
    # rounding of the quotient; z = h2 only its own
    b = project_forward_error_bound(X, [0, 1], np.eye(4)[None])
    np.testing.assert_allclose(b, [[2 * g4 + u, 2 * g4 + u, g4]], rtol=1e-12, atol=0)
    # h3 = 2 (M33 = 2): x = 1/2, off by (g4 + (1/2) 2 g4) / 2 + u / 2
    M2 = np.diag([1.0, 1.0, 1.0, 2.0])[None]
    b = project_forward_error_bound(X, [0, 1], M2)
    np.testing.assert_allclose(b, [[g4 + u / 2, g4 + u / 2, g4]], rtol=1e-12, atol=0)
    # backward with g = (1, 1, 1) through the identity: gh = (1, 1, 1, 2);
    # the errors of gh: g eh3 / h3^2 + u gh for the first two, 0 for the
    # third, (g0 e_x + g1 e_y) / h3 + gh3 (eh3 / h3 + 4u) for the fourth
    bv, bm = project_backward_error_bound(X, [0, 1], np.eye(4)[None], np.ones((1, 3)))
    dgh = np.array([g4 + u, g4 + u, 0.0, 2 * (2 * g4 + u) + 2 * (g4 + 4 * u)])
    gh = np.array([1.0, 1.0, 1.0, 2.0])
    # vertex entry c: sum_r |M_rc| (dgh_r + g4 gh_r), doubled
    np.testing.assert_allclose(bv, 2 * (dgh[:3] + g4 * gh[:3])[None], rtol=1e-12, atol=0)
    # camera entry (r, c): (dgh_r + u gh_r) |Xh_c| plus one addition (a mesh
    # of one vertex) of u gh_r |Xh_c|, doubled
    np.testing.assert_allclose(bm[0], 2 * np.repeat((dgh + 2 * u * gh)[:, None], 4, axis=1), rtol=1e-12, atol=0)

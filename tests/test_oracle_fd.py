"""Backward pass of the oracle against central finite differences (binary64).

L = sum over all slots of gz*zbuf + gb.bary + gd*dists with seeded upstream
gradients, on meshes of at most 4 faces at 16x16. A coordinate whose +-h
perturbation changes any discrete state (pix_to_face, the inside flag, a clip
state, the nearest edge or its clamp) is skipped; at least 90% must be
testable.
"""

import numpy as np
import pytest

H = W = 16
STEP = 1e-6


def _scene(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    nf = int(rng.integers(1, 5))
    K = int(rng.integers(1, 4))
    blur = float(rng.choice([0.0, 1e-3, 1e-2]))
    c = rng.uniform(-0.6, 0.6, (nf, 1, 2))
    xy = c + rng.normal(0.0, 0.35, (nf, 3, 2))
    z = rng.uniform(0.5, 3.0, (nf, 1, 1)) + rng.normal(0.0, 0.3, (nf, 3, 1))
    v = np.concatenate([xy, z], axis=2).reshape(-1, 3)
    faces = np.arange(3 * nf, dtype=np.int64).reshape(nf, 3)
    if nf >= 2 and rng.random() < 0.5:
        faces[1, 0] = faces[0, 1]  # a shared vertex
    offsets = np.array([0, nf], np.int64)
    g = {
        "zbuf": rng.standard_normal((1, H, W, K)),
        "bary": rng.standard_normal((1, H, W, K, 3)),
        "dists": rng.standard_normal((1, H, W, K)) * 10,
    }
    return v.astype(np.float64), faces, offsets, K, blur, g


def _loss(oracle, v, f, o, K, blur, g):
    p2f, zb, ba, di, st = oracle.rasterize(v, f, o, H, W, K, blur, precision="f64", with_state=True)
    L = (g["zbuf"] * zb).sum() + (g["bary"] * ba).sum() + (g["dists"] * di).sum()
    return L, p2f, st


@pytest.mark.parametrize("seed", list(range(12)))
def test_backward_matches_finite_differences(oracle_mod, seed):
    v, f, o, K, blur, g = _scene(seed)
    L0, p2f, st = _loss(oracle_mod, v, f, o, K, blur, g)
    grad = oracle_mod.backward(v, f, o, H, W, K, blur, p2f,
                               g["zbuf"].astype(np.float32), g["bary"].astype(np.float32),
                               g["dists"].astype(np.float32), precision="f64")
    # the analytic pass reads float32 upstream gradients; use the same values here
    g32 = {k: a.astype(np.float32).astype(np.float64) for k, a in g.items()}
    used = np.unique(f)
    tested = skipped = 0
    for vi in used:
        for c in range(3):
            vp, vm = v.copy(), v.copy()
            vp[vi, c] += STEP
            vm[vi, c] -= STEP
            Lp, pp, sp = _loss(oracle_mod, vp, f, o, K, blur, g32)
            Lm, pm, sm = _loss(oracle_mod, vm, f, o, K, blur, g32)
            if not (np.array_equal(pp, p2f) and np.array_equal(pm, p2f)
                    and np.array_equal(sp, st) and np.array_equal(sm, st)):
                skipped += 1
                continue
            fd = (Lp - Lm) / (2 * STEP)
            an = grad[vi, c]
            assert abs(fd - an) <= 1e-5 * (1 + abs(an)), (vi, c, fd, an)
            tested += 1
    assert tested >= 0.9 * (tested + skipped), (tested, skipped)
    assert np.abs(grad).max() > 0


def test_finite_differences_catch_a_wrong_gradient(oracle_mod):
    """The check above is sensitive: a deliberately perturbed analytic gradient
    on one coordinate must fail it."""
    v, f, o, K, blur, g = _scene(3)
    L0, p2f, st = _loss(oracle_mod, v, f, o, K, blur, g)
    grad = oracle_mod.backward(v, f, o, H, W, K, blur, p2f, g["zbuf"].astype(np.float32),
                               g["bary"].astype(np.float32), g["dists"].astype(np.float32),
                               precision="f64")
    g32 = {k: a.astype(np.float32).astype(np.float64) for k, a in g.items()}
    vi, c = int(f[0, 0]), 0
    vp, vm = v.copy(), v.copy()
    vp[vi, c] += STEP
    vm[vi, c] -= STEP
    fd = (_loss(oracle_mod, vp, f, o, K, blur, g32)[0] - _loss(oracle_mod, vm, f, o, K, blur, g32)[0]) / (2 * STEP)
    assert abs(fd - grad[vi, c]) <= 1e-5 * (1 + abs(grad[vi, c]))
    assert abs(fd - 1.01 * grad[vi, c]) > 1e-5 * (1 + abs(grad[vi, c])) or abs(grad[vi, c]) < 1e-3

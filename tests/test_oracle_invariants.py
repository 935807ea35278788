"""Invariants that the definition fixes, checked on the oracle over seeded
workloads (a full icosphere image, a heterogeneous batch with an empty mesh,
a triangle soup and K=50 soups with culled faces and blur)."""

import numpy as np
import pytest

from workloads import make_workload

WORKLOADS = ["sphere64", "small_hetero", "small_soup", "small_soups"]


@pytest.fixture(scope="module")
def runs(oracle_mod):
    out = {}
    for name in WORKLOADS:
        w = make_workload(name)
        res = oracle_mod.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, with_state=True)
        out[name] = (w, res)
    return out


@pytest.mark.parametrize("name", WORKLOADS)
def test_slot_invariants(runs, name):
    w, (p2f, zbuf, bary, dists, state) = runs[name]
    filled = p2f >= 0
    assert filled.any()
    # padding is a contiguous suffix holding exactly -1 everywhere
    assert np.all(np.diff(filled.astype(np.int8), axis=-1) <= 0)
    assert np.all(zbuf[~filled] == -1) and np.all(dists[~filled] == -1) and np.all(bary[~filled] == -1)
    # faces belong to the pixel's own mesh
    n_idx = np.arange(w.N)[:, None, None, None]
    lo = w.offsets[:-1][n_idx] + 0 * p2f
    hi = w.offsets[1:][n_idx] + 0 * p2f
    assert np.all((p2f[filled] >= lo[filled]) & (p2f[filled] < hi[filled]))
    # clipped, renormalised barycentrics: in [0,1], summing to 1
    b = bary[filled].astype(np.float64)
    assert np.all((b >= 0) & (b <= 1))
    assert np.max(np.abs(b.sum(-1) - 1)) <= 5e-7
    # zbuf is the barycentric interpolation of the vertex depths, and > 0
    fz = w.verts[w.faces[p2f[filled]]][..., 2].astype(np.float64)
    zi = (b * fz).sum(-1)
    assert np.max(np.abs(zi - zbuf[filled]) / (1 + np.abs(zi))) <= 1e-6
    assert np.all(zbuf[filled] > 0)
    # ascending (z, face) along the K axis
    z2, f2 = zbuf[..., 1:], p2f[..., 1:]
    z1, f1 = zbuf[..., :-1], p2f[..., :-1]
    both = (f2 >= 0)
    assert np.all((z1[both] < z2[both]) | ((z1[both] == z2[both]) & (f1[both] < f2[both])))
    # sign of dists is the strict-inside test; outside slots lie within blur
    inside = (state[filled] & 1) == 1
    d = dists[filled]
    assert np.array_equal(d < 0, inside)
    assert np.all(inside | (d < np.float32(w.blur)))


@pytest.mark.parametrize("name", ["small_hetero", "small_soups"])
def test_prefix_property(oracle_mod, runs, name):
    w, (p2f, zbuf, bary, dists, _) = runs[name]
    for K2 in (1, w.K // 2):
        q = oracle_mod.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, K2, w.blur)
        for a, b in zip(q, (p2f, zbuf, bary, dists)):
            np.testing.assert_array_equal(a, b[:, :, :, :K2])


def test_batch_is_concatenation_of_single_meshes(oracle_mod, runs):
    w, full = runs["small_hetero"]
    for n in range(w.N):
        f0, f1 = int(w.offsets[n]), int(w.offsets[n + 1])
        single = oracle_mod.rasterize(w.verts, w.faces[f0:f1], np.array([0, f1 - f0]),
                                      w.H, w.W, w.K, w.blur)
        p = single[0].copy()
        p[p >= 0] += f0
        np.testing.assert_array_equal(p[0], full[0][n])
        for a, b in zip(single[1:], full[1:4]):
            np.testing.assert_array_equal(a[0], b[n])


def test_blur_monotone_candidate_sets(oracle_mod):
    w = make_workload("small_soups")
    pix = np.arange(0, w.pixels, 97)
    Kall = int(np.diff(w.offsets).max())
    sets = []
    for blur in (0.0, 1e-4, 1e-3, 4e-3):
        p = oracle_mod.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, Kall, blur, pixels=pix)[0]
        sets.append([set(r[r >= 0].tolist()) for r in p])
    for a, b in zip(sets, sets[1:]):
        assert all(x <= y for x, y in zip(a, b))
    assert sum(len(s) for s in sets[-1]) > sum(len(s) for s in sets[0])


def test_face_permutation_within_mesh(oracle_mod):
    w = make_workload("small_soups")
    rng = np.random.Generator(np.random.PCG64(5))
    perm = np.arange(w.F)
    for n in range(w.N):
        f0, f1 = int(w.offsets[n]), int(w.offsets[n + 1])
        perm[f0:f1] = f0 + rng.permutation(f1 - f0)
    base = oracle_mod.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur)
    perm_out = oracle_mod.rasterize(w.verts, w.faces[perm], w.offsets, w.H, w.W, w.K, w.blur)
    mapped = np.where(perm_out[0] >= 0, perm[np.maximum(perm_out[0], 0)], -1)
    # identical except where equal depths reorder
    diff = mapped != base[0]
    np.testing.assert_array_equal(perm_out[1], base[1])  # the depth sequence never changes
    if diff.any():
        zt = base[1][diff]
        assert np.all(zt >= 0)


def test_zbuf_gradient_sums_to_upstream(oracle_mod, runs):
    """d zbuf / d z_k = bary_k and the barycentrics sum to 1, so the z
    components of grad_verts add up to the upstream zbuf gradient over filled
    slots."""
    w, (p2f, zbuf, bary, dists, _) = runs["small_hetero"]
    rng = np.random.Generator(np.random.PCG64(11))
    gz = rng.standard_normal(p2f.shape).astype(np.float32)
    g = oracle_mod.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, p2f, grad_zbuf=gz)
    total = gz[p2f >= 0].astype(np.float64).sum()
    assert abs(g[:, 2].sum() - total) <= 1e-5 * (1 + np.abs(gz[p2f >= 0]).sum())
    assert np.all(np.isfinite(g))


def test_binary64_drift_is_small(oracle_mod, runs):
    """The binary32 canonical evaluation and the binary64 one agree on almost
    every face list. Values agree to binary32 rounding except on slivers
    (nearly edge-on faces), where the barycentrics of a pixel next to the face
    are ill-conditioned: their binary32 error grows like eps / |A|."""
    w, (p2f, zbuf, bary, dists, _) = runs["small_hetero"]
    q = oracle_mod.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, precision="f64")
    same = (q[0] == p2f)
    assert same.all(axis=-1).mean() > 0.999
    m = same & (p2f >= 0)
    err = np.abs(q[2] - bary).max(-1)
    assert np.median(err[m]) < 1e-6
    v = w.verts.astype(np.float64)[w.faces[p2f[m]]]
    A = np.abs((v[:, 1, 0] - v[:, 0, 0]) * (v[:, 2, 1] - v[:, 0, 1])
               - (v[:, 1, 1] - v[:, 0, 1]) * (v[:, 2, 0] - v[:, 0, 0]))
    bound = 1e-5 + 64 * np.finfo(np.float32).eps * 1e-3 / A
    assert np.all(err[m] <= bound)
    assert np.all(np.abs(q[1][m] - zbuf[m]) <= 3 * bound)

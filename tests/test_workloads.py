"""Seeded input generators: determinism, sizes and value ranges."""

import hashlib

import numpy as np
import pytest

from workloads import icosphere, make_workload, sample_pixels, upstream_grads


def _digest(w):
    h = hashlib.sha256()
    for a in (w.verts, w.faces, w.offsets):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("L", [0, 1, 2, 3, 4])
def test_icosphere_counts(L):
    v, f = icosphere(L)
    assert v.shape == (10 * 4 ** L + 2, 3)
    assert f.shape == (20 * 4 ** L, 3)
    np.testing.assert_allclose(np.linalg.norm(v, axis=1), 1.0, atol=1e-12)
    # closed 2-manifold: every edge is shared by exactly two faces
    e = np.sort(np.concatenate([f[:, [0, 1]], f[:, [1, 2]], f[:, [2, 0]]]), axis=1)
    _, cnt = np.unique(e, axis=0, return_counts=True)
    assert np.all(cnt == 2)


@pytest.mark.parametrize("name", ["sphere64", "spheres8_137", "small_hetero", "small_soup", "small_soups"])
def test_deterministic_and_well_formed(name):
    a, b = make_workload(name), make_workload(name)
    assert _digest(a) == _digest(b)
    assert a.verts.dtype == np.float32 and a.faces.dtype == np.int64 and a.offsets.dtype == np.int64
    assert a.offsets[0] == 0 and a.offsets[-1] == a.F and np.all(np.diff(a.offsets) >= 0)
    assert a.faces.min() >= 0 and a.faces.max() < a.V
    c = make_workload(name, seed=a.seed + 1)
    assert _digest(c) != _digest(a)


def test_named_sizes():
    w = make_workload("sphere64")
    assert (w.N, w.F, w.V, w.H, w.W, w.K, w.blur) == (1, 320, 162, 64, 64, 1, 0.0)
    assert np.abs(w.verts[:, :2]).max() <= np.float32(0.8)
    assert w.verts[:, 2].min() >= 1.5 - 1e-6 and w.verts[:, 2].max() <= 2.5 + 1e-6
    w = make_workload("spheres8_137")
    assert (w.N, w.F, w.V, w.H, w.W, w.K) == (8, 40960, 20496, 137, 137, 8)
    assert w.blur == float(np.float32(1e-4))
    assert np.array_equal(np.diff(w.offsets), [5120] * 8)


def test_grads_and_samples_are_seeded():
    w = make_workload("sphere64")
    g1, g2 = upstream_grads(w), upstream_grads(w)
    assert g1["bary"] is None and g1["dists"] is None
    np.testing.assert_array_equal(g1["zbuf"], g2["zbuf"])
    p = sample_pixels(w, 100)
    assert np.all(np.diff(p) > 0) and p[0] == 0 and p[-1] == w.pixels - 1

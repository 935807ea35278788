"""The region reduction the dense full-size GPU checks use
(parity.oracle_region: the oracle run on only the faces whose grown box
reaches the region) gives exactly the whole-batch oracle's outputs and
gradients, on every pixel of small workloads split into regions, with the
default settings and with the rasterizer settings."""

import numpy as np
import pytest

import oracle
from parity import oracle_region
from workloads import make_workload, upstream_grads


ALL_SETTINGS = oracle.PERSPECTIVE | oracle.CULL_BACKFACES | oracle.UNCLIPPED_BARY


@pytest.mark.parametrize("name,settings", [("small_hetero", 0), ("small_soups", 0), ("sphere64", 0),
                                           ("small_hetero", ALL_SETTINGS), ("small_soups", oracle.PERSPECTIVE)])
def test_region_oracle_equals_whole_oracle(name, settings):
    w = make_workload(name)
    full = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, settings=settings)
    gr = upstream_grads(w)
    for n in range(w.N):
        for i0 in range(0, w.H, 16):
            for j0 in range(0, w.W, 24):
                i1, j1 = min(w.H, i0 + 16), min(w.W, j0 + 24)
                pix = None
                sel = lambda a: None if a is None else a[n, i0:i1, j0:j1].reshape((-1, w.K) + a.shape[4:])
                pix, got, gv = oracle_region(oracle, w.verts, w.faces, w.offsets, n, w.H, w.W, w.K, w.blur,
                                             i0, i1, j0, j1, grads=(sel(gr["zbuf"]), sel(gr["bary"]),
                                                                    sel(gr["dists"])), settings=settings)
                for a, b in zip(got, full):
                    np.testing.assert_array_equal(a, b[n, i0:i1, j0:j1].reshape(a.shape))
                ref_gv = oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur,
                                         full[0].reshape((-1, w.K))[pix], sel(gr["zbuf"]), sel(gr["bary"]),
                                         sel(gr["dists"]), pixels=pix, settings=settings)
                np.testing.assert_allclose(gv, ref_gv, rtol=0, atol=1e-12 * max(1.0, np.abs(ref_gv).max()))

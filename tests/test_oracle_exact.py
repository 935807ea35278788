"""Binary32 oracle against exact rational brute force on tiny random inputs.

Vertices sit on a grid of multiples of 1/64, so vertex differences and edge
functions are exact in binary32 and the inside decision is exact; the only
roundings are the divisions and what follows them. The oracle must reproduce
the exact K-lists (ties broken by face index, z <= 0 skipped, blur inclusion)
except at near-threshold pixels, and the exact values to 2e-6.
"""

import numpy as np
import pytest

from exact_raster import exact_rasterize
from parity import compare_forward, exact_excuse


def _case(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    H = int(rng.choice([4, 5, 6, 8]))
    W = int(rng.choice([4, 6, 7, 8]))
    K = int(rng.integers(1, 5))
    blur = float(rng.choice([0.0, 1.0 / 64, 0.05]))
    N = int(rng.integers(1, 3))
    verts, faces, offsets = [], [], [0]
    for n in range(N):
        nf = int(rng.integers(1, 7))
        for f in range(nf):
            if f > 0 and rng.random() < 0.2:
                faces.append(faces[-1])  # coincident face: exact depth tie
                offsets[-1] += 0
                continue
            base = len(verts)
            for _ in range(3):
                x = rng.integers(-80, 81) / 64.0
                y = rng.integers(-80, 81) / 64.0
                z = rng.integers(-16, 192) / 64.0
                verts.append((x, y, z))
            if rng.random() < 0.25:  # constant-depth face: ties across faces
                zc = rng.integers(16, 128) / 64.0
                for q in range(3):
                    verts[base + q] = verts[base + q][:2] + (zc,)
            faces.append((base, base + 1, base + 2))
        offsets.append(len(faces))
    return (np.asarray(verts, np.float32), np.asarray(faces, np.int64),
            np.asarray(offsets, np.int64), H, W, K, blur)


@pytest.mark.parametrize("seed", list(range(24)))
def test_oracle_matches_exact(oracle_mod, seed):
    v, f, o, H, W, K, blur = _case(seed)
    exact, details = exact_rasterize(v, f, o, H, W, K, blur)
    got = oracle_mod.rasterize(v, f, o, H, W, K, blur)
    N = len(o) - 1
    rep = compare_forward(exact, got, K, atol=2e-6, excuse=exact_excuse(details, N, H, W, blur))
    assert not rep["unexcused"], rep
    assert len(rep["excused"]) <= max(1, rep["pixels"] // 10), rep
    assert rep["values_ok"], rep
    assert rep["padding_ok"]
    # sign of dists is exactly the strict-inside test, on every matching slot
    p2f = got[0].reshape(-1, K)
    ex_p2f = exact[0].reshape(-1, K)
    dists = got[3].reshape(-1, K)
    for r in range(p2f.shape[0]):
        n, rem = divmod(r, H * W)
        i, j = divmod(rem, W)
        for k in range(K):
            fid = p2f[r, k]
            if fid >= 0 and fid == ex_p2f[r, k]:
                inside = details[(n, i, j)][int(fid)]["inside"]
                assert (dists[r, k] < 0) == inside


def test_exact_cases_have_no_excuses_on_power_of_two_grids(oracle_mod):
    """With power-of-two image sizes the pixel centres are dyadic too; the
    oracle then reproduces every decision of the exact computation."""
    total = 0
    for seed in range(100, 112):
        v, f, o, H, W, K, blur = _case(seed)
        H, W = 8, 8
        exact, details = exact_rasterize(v, f, o, H, W, K, blur)
        got = oracle_mod.rasterize(v, f, o, H, W, K, blur)
        rep = compare_forward(exact, got, K, atol=2e-6,
                              excuse=exact_excuse(details, len(o) - 1, H, W, blur))
        assert not rep["unexcused"]
        total += len(rep["excused"])
    assert total <= 2

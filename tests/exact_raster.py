"""Exact-rational brute force of K-nearest-face rasterization, for tiny inputs.

An independent formulation of the same definition, in Python `Fraction`s:
barycentrics as ratios of exact signed sub-triangle areas, inside as an exact
sign test, point-segment squared distance by the vertex/edge region case
split (|p-a|^2 - s^2/|u|^2 in the edge region) rather than the clamped
projection, exact clipping, renormalisation and depth. Pixel centres are the
binary32 values fl(fl((2j+1)/W) - 1), which is how the library defines them.

It shares nothing with oracle/ except the definition it implements.
"""

from fractions import Fraction as Fr

import numpy as np


def pixel_centre_f32(j: int, W: int) -> Fr:
    v = np.float32(np.float32(2 * j + 1) / np.float32(W)) - np.float32(1)
    return Fr(float(np.float32(v)))


def _cross(ax, ay, bx, by):
    return ax * by - ay * bx


def _seg_d2(px, py, ax, ay, bx, by):
    ux, uy = bx - ax, by - ay
    L = ux * ux + uy * uy
    qx, qy = px - ax, py - ay
    s = qx * ux + qy * uy
    if s <= 0:
        return qx * qx + qy * qy
    if s >= L:
        rx, ry = px - bx, py - by
        return rx * rx + ry * ry
    return qx * qx + qy * qy - s * s / L


def face_at_pixel(P, px, py, blur):
    """P: three (x, y, z) Fractions. Returns dict or None (degenerate)."""
    (x0, y0, z0), (x1, y1, z1), (x2, y2, z2) = P
    A = _cross(x1 - x0, y1 - y0, x2 - x0, y2 - y0)
    if A == 0:
        return None
    a0 = _cross(x1 - px, y1 - py, x2 - px, y2 - py)
    a1 = _cross(x2 - px, y2 - py, x0 - px, y0 - py)
    a2 = _cross(x0 - px, y0 - py, x1 - px, y1 - py)
    b = [a0 / A, a1 / A, a2 / A]
    inside = all(bk > 0 for bk in b)
    d2 = min(_seg_d2(px, py, x0, y0, x1, y1), _seg_d2(px, py, x1, y1, x2, y2),
             _seg_d2(px, py, x2, y2, x0, y0))
    c = [min(max(bk, Fr(0)), Fr(1)) for bk in b]
    S = c[0] + c[1] + c[2]
    bh = [ck / S for ck in c]
    z = bh[0] * z0 + bh[1] * z1 + bh[2] * z2
    included = inside or d2 < blur
    return {"inside": inside, "d2": d2, "bh": bh, "z": z, "included": included,
            "candidate": included and z > 0}


def exact_rasterize(verts, faces, offsets, H, W, K, blur):
    """Returns (pix_to_face, zbuf, bary, dists) as float64 arrays of the exact
    values, plus details[n][i][j] = list of per-face dicts for the mesh."""
    verts = np.asarray(verts, np.float32)
    blur = Fr(float(np.float32(blur)))
    V = verts.shape[0]
    N = len(offsets) - 1
    p2f = -np.ones((N, H, W, K), np.int64)
    zbuf = -np.ones((N, H, W, K), np.float64)
    bary = -np.ones((N, H, W, K, 3), np.float64)
    dists = -np.ones((N, H, W, K), np.float64)
    details = {}
    for n in range(N):
        for i in range(H):
            py = pixel_centre_f32(i, H)
            for j in range(W):
                px = pixel_centre_f32(j, W)
                per_face = {}
                cands = []
                for f in range(int(offsets[n]), int(offsets[n + 1])):
                    idx = [int(v) for v in faces[f]]
                    if any(v < 0 or v >= V for v in idx):
                        continue
                    P = [tuple(Fr(float(c)) for c in verts[v]) for v in idx]
                    r = face_at_pixel(P, px, py, blur)
                    if r is None:
                        continue
                    per_face[f] = r
                    if r["candidate"]:
                        cands.append((r["z"], f))
                cands.sort()
                details[(n, i, j)] = per_face
                for k, (z, f) in enumerate(cands[:K]):
                    r = per_face[f]
                    p2f[n, i, j, k] = f
                    zbuf[n, i, j, k] = float(z)
                    bary[n, i, j, k] = [float(x) for x in r["bh"]]
                    dists[n, i, j, k] = float(-r["d2"] if r["inside"] else r["d2"])
    return (p2f, zbuf, bary, dists), details

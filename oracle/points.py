"""CPU oracle of point-cloud rasterization: for every pixel, the K nearest
points of its own cloud within a radius, and the backward pass to the point
positions (numpy).

TEST INFRASTRUCTURE ONLY: the plain, slow definition the GPU point
rasterizer is checked against. Only tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py may import this module; it imports nothing
from the GPU package.

The pages list point clouds among the 3D data the renderer handles, next to
meshes (rocketrecap summary, "2:02 Data Structures and I/O"; gptget.net
summary, "Methodology"), with the same per-pixel K-nearest selection and
heterogeneous batching as the mesh rasterizer. They give no formula; the
reading used here, for cloud n owning points [offsets[n], offsets[n+1]) and
pixel (i, j) of image n with centre (px, py) as for meshes:

  candidate      point q with z_q > 0 and d2 = (px - x_q)^2 + (py - y_q)^2 < r2,
                 r2 = radius * radius (binary32), strict;
  order          the K smallest (z_q, q), ascending;
  outputs        idx [N,H,W,K] int64 (global point index), zbuf = z_q,
                 dists = d2; -1 on padding.

With precision 'f32' every operation is one binary32 operation in the
order written (numpy applies no contraction), so decisions and values are
exactly those of a binary32 implementation that follows the same order.

Backward: zbuf = z_q gives dL/dz_q += g_z; dists = d2 gives
dL/dx_q += -2 (px - x_q) g_d and dL/dy_q += -2 (py - y_q) g_d.
"""

from __future__ import annotations

import numpy as np


def _centres(n, dt):
    j = np.arange(n)
    return (np.asarray(2 * j + 1, dt) / dt(n)) - dt(1)


def rasterize_points(points, offsets, H, W, K, radius, precision="f32", pixels=None):
    """points [P,3] (x, y NDC, z depth), offsets [N+1]. Returns (idx, zbuf,
    dists) shaped [N,H,W,K] (or [len(pixels), K] for a list of flat pixel
    ids n*H*W + i*W + j)."""
    dt = np.float32 if precision == "f32" else np.float64
    pts = np.asarray(points, dt).reshape(-1, 3)
    off = np.asarray(offsets, np.int64)
    N = len(off) - 1
    r2 = dt(radius) * dt(radius)
    xs, ys = _centres(W, dt), _centres(H, dt)
    pix = np.arange(N * H * W) if pixels is None else np.asarray(pixels, np.int64).reshape(-1)
    idx = np.full((len(pix), K), -1, np.int64)
    zb = np.full((len(pix), K), -1, dt)
    ds = np.full((len(pix), K), -1, dt)
    for n in range(N):
        sel = np.nonzero(pix // (H * W) == n)[0]
        lo, hi = int(off[n]), int(off[n + 1])
        if len(sel) == 0 or hi <= lo:
            continue
        q = pts[lo:hi]
        rem = pix[sel] % (H * W)
        px = xs[rem % W][:, None]
        py = ys[rem // W][:, None]
        dx = px - q[None, :, 0]
        dy = py - q[None, :, 1]
        d2 = dx * dx + dy * dy
        cand = (d2 < r2) & (q[None, :, 2] > 0)
        for a, row in enumerate(sel):
            c = np.nonzero(cand[a])[0]
            if len(c) == 0:
                continue
            order = np.lexsort((c, q[c, 2]))[:K]   # by z, then index
            c = c[order]
            m = len(c)
            idx[row, :m] = lo + c
            zb[row, :m] = q[c, 2]
            ds[row, :m] = d2[a, c]
    if pixels is None:
        shape = (N, H, W, K)
        return idx.reshape(shape), zb.reshape(shape), ds.reshape(shape)
    return idx, zb, ds


def rasterize_points_backward(points, offsets, H, W, K, idx, grad_zbuf=None, grad_dists=None, pixels=None,
                              precision="f32"):
    """grad_points [P,3] (binary64 sums of the per-slot terms) from the
    gradients of zbuf and dists (either may be None); the pixel centres are
    those of the forward pass of the same precision."""
    pts = np.asarray(points, np.float64).reshape(-1, 3)
    N = len(offsets) - 1
    pix = np.arange(N * H * W) if pixels is None else np.asarray(pixels, np.int64).reshape(-1)
    idx = np.asarray(idx).reshape(len(pix), K)
    gz = None if grad_zbuf is None else np.asarray(grad_zbuf, np.float64).reshape(len(pix), K)
    gd = None if grad_dists is None else np.asarray(grad_dists, np.float64).reshape(len(pix), K)
    out = np.zeros_like(pts)
    rem = pix % (H * W)
    dt = np.float32 if precision == "f32" else np.float64
    px = _centres(W, dt).astype(np.float64)[rem % W]
    py = _centres(H, dt).astype(np.float64)[rem // W]
    for k in range(K):
        m = idx[:, k] >= 0
        q = idx[m, k]
        if gz is not None:
            np.add.at(out[:, 2], q, gz[m, k])
        if gd is not None:
            np.add.at(out[:, 0], q, -2.0 * (px[m] - pts[q, 0]) * gd[m, k])
            np.add.at(out[:, 1], q, -2.0 * (py[m] - pts[q, 1]) * gd[m, k])
    return out

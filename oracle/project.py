"""CPU oracle of the upstream projection: world-space vertices of a packed
batch of meshes to the screen space the rasterizer takes (x, y in NDC,
z = depth), and its backward pass (binary64 numpy).

TEST INFRASTRUCTURE ONLY: the plain, slow definition the GPU projection is
checked against. Only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import this module; it imports nothing from the GPU
package.

The pages put the renderer between 3D model parameters and 2D pixels and
differentiate through it from pixels back to the 3D parameters (rocketrecap
summary, "3:52 Differentiable Renderer"), with several viewpoints per object
(the same summary, "22:00 2D-to-3D Reconstruction"). They give no camera
model. The reading used here: mesh n is seen through one 4x4 matrix M_n
(row-major); for a vertex X of mesh n, h = M_n (X, 1) and

    x_ndc = h0 / h3,   y_ndc = h1 / h3,   z = h2

(perspective division of x and y; the third row gives the depth the
rasterizer interpolates, e.g. the view depth). Mesh n owns vertices
[vert_offsets[n], vert_offsets[n+1]).

Backward: with upstream gradient g = dL/d(x_ndc, y_ndc, z),
    dL/dh0 = g0 / h3, dL/dh1 = g1 / h3, dL/dh2 = g2,
    dL/dh3 = -(g0 h0 + g1 h1) / h3^2,
    dL/dX = M_n[:, :3]^T dL/dh,   dL/dM_n += dL/dh (X, 1)^T over the mesh's vertices.
"""

from __future__ import annotations

import numpy as np


def _mesh_of_vertex(vert_offsets, V):
    off = np.asarray(vert_offsets, np.int64)
    return np.repeat(np.arange(len(off) - 1), np.diff(off))[:V]


def project_forward(verts, vert_offsets, cameras):
    """verts [V,3], vert_offsets [N+1], cameras [N,4,4] -> [V,3] (x_ndc, y_ndc, z)."""
    X = np.asarray(verts, np.float64)
    M = np.asarray(cameras, np.float64)
    mesh = _mesh_of_vertex(vert_offsets, X.shape[0])
    Xh = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
    h = np.einsum("vrc,vc->vr", M[mesh], Xh)
    return np.stack([h[:, 0] / h[:, 3], h[:, 1] / h[:, 3], h[:, 2]], axis=1)


def project_backward(verts, vert_offsets, cameras, grad_out):
    """(grad_verts [V,3], grad_cameras [N,4,4]) from grad_out [V,3]."""
    X = np.asarray(verts, np.float64)
    M = np.asarray(cameras, np.float64)
    g = np.asarray(grad_out, np.float64)
    mesh = _mesh_of_vertex(vert_offsets, X.shape[0])
    Xh = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
    h = np.einsum("vrc,vc->vr", M[mesh], Xh)
    gh = np.stack([g[:, 0] / h[:, 3], g[:, 1] / h[:, 3], g[:, 2],
                   -(g[:, 0] * h[:, 0] + g[:, 1] * h[:, 1]) / (h[:, 3] * h[:, 3])], axis=1)
    gX = np.einsum("vrc,vr->vc", M[mesh][:, :, :3], gh)
    gM = np.zeros_like(M)
    np.add.at(gM, mesh, gh[:, :, None] * Xh[:, None, :])
    return gX, gM


def project_forward_error_bound(verts, vert_offsets, cameras):
    """First-order bound on |binary32 result - exact| for binary32 inputs
    evaluated with each h_r a sum of four rounded products and one correctly
    rounded division: with u = 2^-24, |dh_r| <= gamma_4 sum_c |M_rc X_c|, and
    the quotient adds the errors of both operands plus one rounding."""
    X = np.asarray(verts, np.float64)
    M = np.asarray(cameras, np.float64)
    mesh = _mesh_of_vertex(vert_offsets, X.shape[0])
    Xh = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
    Mm = M[mesh]
    h = np.einsum("vrc,vc->vr", Mm, Xh)
    a = np.einsum("vrc,vc->vr", np.abs(Mm), np.abs(Xh))
    u = 2.0 ** -24
    eh = 4 * u * a / (1 - 4 * u)   # gamma_4: four products summed (inputs exact in binary32)
    q0, q1 = h[:, 0] / h[:, 3], h[:, 1] / h[:, 3]
    e0 = (eh[:, 0] + np.abs(q0) * eh[:, 3]) / np.abs(h[:, 3]) + u * np.abs(q0)
    e1 = (eh[:, 1] + np.abs(q1) * eh[:, 3]) / np.abs(h[:, 3]) + u * np.abs(q1)
    return np.stack([e0, e1, eh[:, 2]], axis=1)


def project_backward_error_bound(verts, vert_offsets, cameras, grad_out, cam_sum_depth=None):
    """First-order bounds on |binary32 result - exact| of the backward pass
    for binary32 inputs, evaluated as: gh = (g0 / h3, g1 / h3, g2,
    -(g0 x + g1 y) / h3) with the binary32 x, y of the forward pass; each
    vertex gradient entry a sum of four rounded products; each camera entry
    a sum of the rounded products gh_r X_c in which every term passes
    through at most cam_sum_depth[n] rounded additions (default: V_n, a
    plain running sum; a tree or a mix of running sums and trees has less).

    The inputs' own error: h_r is off by eh_r = gamma_4 sum_c |M_rc X_c|, so
    g_k / h3 moves by |g_k| eh3 / h3^2 and the x, y the last component uses
    by their forward bounds. Returns (bound_verts [V,3], bound_cameras
    [N,4,4]), each doubled to cover second-order terms."""
    X = np.asarray(verts, np.float64)
    M = np.asarray(cameras, np.float64)
    g = np.abs(np.asarray(grad_out, np.float64))
    off = np.asarray(vert_offsets, np.int64)
    mesh = _mesh_of_vertex(off, X.shape[0])
    Xh = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
    Mm = M[mesh]
    h = np.einsum("vrc,vc->vr", Mm, Xh)
    a = np.einsum("vrc,vc->vr", np.abs(Mm), np.abs(Xh))
    u = 2.0 ** -24
    g4 = 4 * u / (1 - 4 * u)
    eh = g4 * a
    ah3 = np.abs(h[:, 3])
    q0, q1 = np.abs(h[:, 0] / h[:, 3]), np.abs(h[:, 1] / h[:, 3])
    eq = project_forward_error_bound(verts, vert_offsets, cameras)
    gh = np.stack([g[:, 0] / ah3, g[:, 1] / ah3, g[:, 2], (g[:, 0] * q0 + g[:, 1] * q1) / ah3], axis=1)
    dgh = np.stack([
        g[:, 0] * eh[:, 3] / ah3 ** 2 + u * gh[:, 0],
        g[:, 1] * eh[:, 3] / ah3 ** 2 + u * gh[:, 1],
        np.zeros(len(X)),
        (g[:, 0] * eq[:, 0] + g[:, 1] * eq[:, 1]) / ah3 + gh[:, 3] * (eh[:, 3] / ah3 + 4 * u),
    ], axis=1)
    bound_v = np.einsum("vrc,vr->vc", np.abs(Mm[:, :, :3]), dgh + g4 * gh)
    depth = np.diff(off).astype(np.float64) if cam_sum_depth is None else np.asarray(cam_sum_depth, np.float64)
    per = (dgh + u * gh)[:, :, None] * np.abs(Xh)[:, None, :]
    tot = gh[:, :, None] * np.abs(Xh)[:, None, :]
    bound_m = np.zeros_like(M)
    np.add.at(bound_m, mesh, per)
    sum_abs = np.zeros_like(M)
    np.add.at(sum_abs, mesh, tot)
    bound_m += (depth * u)[:, None, None] * sum_abs
    return 2 * bound_v, 2 * bound_m

"""Upstream projection on the GPU (through the C ABI) against its oracle.

Every element of the forward pass, the vertex gradient and the camera
gradient must lie within the binary32 error bounds of the stated operation
order (oracle/project.py: project_forward_error_bound,
project_backward_error_bound). The camera entries are summed in 16 slices
per mesh, each a running sum per lane over its share of the slice, a 64-lane
tree, a sum over the four waves, and the 16 slice sums added with atomics in
any order: a term passes at most ceil(ceil(V_n / 16) / 256) + 6 + 3 + 16
rounded additions."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, require_gpu, say, to_dev
from oracle.project import (project_backward, project_backward_error_bound, project_forward,
                            project_forward_error_bound)
from workloads import make_workload, projection_inputs, projection_upstream_grads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dmr():
    return require_gpu()


def _run(dmr, X, vo, M, g, want_cams=True):
    Xd, vod, Md, gd = to_dev(X), to_dev(vo), to_dev(M), to_dev(g)
    out = torch.empty_like(Xd)
    dmr.dmr_project_fwd(Xd, vod, Md, out)
    gv = torch.empty_like(Xd)
    gc = torch.empty_like(Md) if want_cams else None
    dmr.dmr_project_bwd(Xd, vod, Md, gd, gv, gc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), gv.cpu().numpy(), None if gc is None else gc.cpu().numpy()


def _check(X, vo, M, g, out, gv, gc):
    ref = project_forward(X, vo, M)
    bound = project_forward_error_bound(X, vo, M)
    err = np.abs(out.astype(np.float64) - ref)
    assert (err <= bound).all(), float((err / bound).max())
    rgx, rgm = project_backward(X, vo, M, g)
    sizes = np.diff(np.asarray(vo, np.int64))
    depth = np.ceil(np.ceil(sizes / 16) / 256) + 6 + 3 + 16
    bv, bm = project_backward_error_bound(X, vo, M, g, cam_sum_depth=depth)
    ev = np.abs(gv - rgx)
    assert (ev <= bv).all(), float((ev / bv).max())
    if gc is not None:
        ec = np.abs(gc - rgm)
        assert (ec <= bm + 1e-30).all(), float((ec / (bm + 1e-30)).max())


@pytest.mark.parametrize("name", ["sphere64", "small_hetero", "hetero16_256", "soups32_512"])
def test_project_workload(dmr, name):
    w = make_workload(name)
    X, vo, M = projection_inputs(w)
    g = projection_upstream_grads(w)
    say(f"[gpu] project {name} V={w.V} N={w.N}")
    out, gv, gc = _run(dmr, X, vo, M, g)
    _check(X, vo, M, g, out, gv, gc)
    # and the projection gives back the rasterizer's screen-space vertices
    assert np.abs(out - w.verts).max() < 1e-4


def test_project_edge_cases(dmr):
    # empty meshes, a mesh of one vertex, a partial last workgroup, meshes
    # that start inside a workgroup, no camera gradient requested
    rng = np.random.default_rng(5)
    sizes = [0, 300, 1, 0, 257, 5, 0]
    vo = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    V, N = int(vo[-1]), len(sizes)
    X = rng.normal(size=(V, 3)).astype(np.float32)
    X[:, 2] += 5.0
    M = rng.normal(0, 0.2, (N, 4, 4)).astype(np.float32)
    for n in range(N):
        M[n, 0, 0] += 2.0
        M[n, 1, 1] += 2.0
        M[n, 2, 2] += 1.0
        M[n, 3, 2] += 1.0
    g = rng.normal(size=(V, 3)).astype(np.float32)
    say("[gpu] project edge cases")
    out, gv, gc = _run(dmr, X, vo, M, g)
    _check(X, vo, M, g, out, gv, gc)
    assert np.all(gc[[0, 3, 6]] == 0)
    out2, gv2, none = _run(dmr, X, vo, M, g, want_cams=False)
    assert none is None
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(gv2, gv)


def test_project_then_rasterize_autograd(dmr):
    # world-space vertices through the projection and the rasterizer: the
    # vertex gradient is the projection's backward of the rasterizer's
    import oracle

    w = make_workload("small_hetero")
    X, vo, M = projection_inputs(w)
    Xd = to_dev(X).requires_grad_(True)
    Md = to_dev(M).requires_grad_(True)
    screen = dmr.project_meshes(Xd, to_dev(vo), Md)
    p2f, zbuf, bary, dists = dmr.rasterize_meshes(screen, to_dev(w.faces), to_dev(w.offsets), (w.H, w.W), w.K,
                                                  w.blur)
    gz = torch.randn(zbuf.shape, generator=torch.Generator().manual_seed(3)).to(DEV)
    (zbuf * gz).sum().backward()
    s = screen.detach().cpu().numpy()
    ref_p2f = oracle.rasterize(s, w.faces, w.offsets, w.H, w.W, w.K, w.blur)[0]
    np.testing.assert_array_equal(p2f.cpu().numpy(), ref_p2f)
    gs = oracle.backward(s, w.faces, w.offsets, w.H, w.W, w.K, w.blur, ref_p2f, gz.cpu().numpy(), None, None)
    rgx, rgm = project_backward(X, vo, M, gs)
    gx = Xd.grad.cpu().numpy()
    assert np.linalg.norm(gx - rgx) <= 1e-4 * np.linalg.norm(rgx)
    assert np.linalg.norm(Md.grad.cpu().numpy() - rgm) <= 1e-4 * np.linalg.norm(rgm)

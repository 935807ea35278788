"""Second-stage blend on the GPU (through the C ABI) against its oracle.

The GPU rasterizes each workload; both sides then blend the very same
rasterizer outputs (copied to the host for the oracle), so this checks the
blend alone. The GPU computes in binary32 with the device exp, the oracle in
binary64: rgba must agree within 1e-4 absolute (alpha within 1e-5). The
exponent of a colour weight is a depth difference scaled by
1/((zfar - znear) gamma), about 1e2-1e4 here, so binary32 rounding of the
depths moves a weight by up to ~1e-4 relative. Each gradient element must
agree within 1e-3 times the sum of the absolute values of the terms it adds
up (blend_backward_scale; the terms cancel exactly for a pixel with a single
face, leaving binary32 noise times 1/sigma), and within 1e-3 relative L2 of
that scale over the image."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, GpuCase, require_gpu, say, to_dev
from oracle.blend import BlendParams, blend_backward, blend_backward_scale, blend_forward
from workloads import blend_upstream_grads, face_colors, make_workload, sample_pixels

pytestmark = pytest.mark.gpu

PARAMS = {
    "sharp": BlendParams(sigma=1e-4, gamma=1e-4, znear=1.0, zfar=100.0, eps=1e-10, background=(1.0, 1.0, 1.0)),
    "soft_near_bg": BlendParams(sigma=1e-3, gamma=2e-2, znear=0.5, zfar=4.0, eps=1e-3, background=(0.2, 0.4, 0.9)),
}


@pytest.fixture(scope="module")
def dmr():
    return require_gpu()


def _gpu_params(dmr, prm):
    return dmr.blend_params(prm.sigma, prm.gamma, prm.znear, prm.zfar, prm.eps, prm.background)


def _blend_gpu(dmr, p2f, zbuf, dists, colors_t, prm, grad_rgba=None):
    shape = tuple(p2f.shape[:-1])
    rgba = torch.empty(shape + (4,), dtype=torch.float32, device=DEV)
    dmr.dmr_blend_fwd(p2f, zbuf, dists, colors_t, _gpu_params(dmr, prm), rgba)
    gz = gd = None
    if grad_rgba is not None:
        gz = torch.empty_like(zbuf)
        gd = torch.empty_like(dists)
        dmr.dmr_blend_bwd(p2f, zbuf, dists, colors_t, _gpu_params(dmr, prm), grad_rgba, gz, gd)
    torch.cuda.synchronize()
    return rgba, gz, gd


def _check(ref_rgba, got_rgba, ref_g=None, got_g=None, scales=None):
    np.testing.assert_allclose(got_rgba[..., :3], ref_rgba[..., :3], atol=1e-4, rtol=0)
    np.testing.assert_allclose(got_rgba[..., 3], ref_rgba[..., 3], atol=1e-5, rtol=0)
    if ref_g is not None:
        for r, g, sc in zip(ref_g, got_g, scales):
            err = np.abs(g.astype(np.float64) - r)
            assert (err <= 1e-3 * sc + 1e-12).all(), float((err / (sc + 1e-30)).max())
            assert np.linalg.norm(err) <= 1e-3 * max(np.linalg.norm(sc), 1e-30)


# A sigma far below the blur radius: outside faces get coverage weights that
# underflow binary32 (exp(-d / sigma) with d / sigma up to 333 at a blur
# radius of 1e-4, and 3333 at 1e-3, where they underflow binary64 too), so a
# pixel reached only by such faces has every weight, and a far background,
# below the smallest float. Both sides sum in the log domain and must still
# give the ratio.
VERY_SHARP = BlendParams(sigma=3e-7, gamma=1e-5, znear=1.0, zfar=100.0, eps=1e-10, background=(0.3, 0.6, 0.1))


@pytest.mark.parametrize("pname", list(PARAMS) + ["very_sharp"])
@pytest.mark.parametrize("name", ["sphere64", "spheres8_137", "small_hetero", "small_soups"])
def test_blend_full_image(dmr, name, pname):
    w = make_workload(name)
    prm = VERY_SHARP if pname == "very_sharp" else PARAMS[pname]
    say(f"[gpu] blend {name} {pname}")
    g = GpuCase.from_workload(w)
    p2f, zbuf, _, dists = g.forward()
    colors = face_colors(w)
    grad = blend_upstream_grads(w)
    rgba, gz, gd = _blend_gpu(dmr, p2f, zbuf, dists, to_dev(colors), prm, to_dev(grad))
    hp, hz, hd = p2f.cpu().numpy(), zbuf.cpu().numpy(), dists.cpu().numpy()
    ref = blend_forward(hp, hz, hd, colors, prm)
    rz, rd = blend_backward(hp, hz, hd, colors, prm, grad)
    sc = blend_backward_scale(hp, hz, hd, colors, prm, grad)
    got = rgba.cpu().numpy()
    assert np.isfinite(got).all() and np.isfinite(ref).all()
    _check(ref, got, (rz, rd), (gz.cpu().numpy(), gd.cpu().numpy()), sc)


@pytest.mark.parametrize("name,n", [("hetero16_256", 20000), ("soups32_512", 5000)])
def test_blend_full_size_sampled(dmr, name, n):
    # soups32_512 has K = 50: four slot chunks per pixel (16, 16, 16, 2)
    w = make_workload(name)
    prm = PARAMS["sharp"]
    say(f"[gpu] blend {name} sampled")
    g = GpuCase.from_workload(w)
    p2f, zbuf, _, dists = g.forward()
    colors = face_colors(w)
    grad = blend_upstream_grads(w)
    rgba, gz, gd = _blend_gpu(dmr, p2f, zbuf, dists, to_dev(colors), prm, to_dev(grad))
    pix = sample_pixels(w, n)
    idx = torch.from_numpy(pix).to(DEV)
    K = w.K
    sel = lambda t, tail: t.reshape((-1,) + tail).index_select(0, idx).cpu().numpy()
    hp, hz, hd = sel(p2f, (K,)), sel(zbuf, (K,)), sel(dists, (K,))
    ref = blend_forward(hp, hz, hd, colors, prm)
    gs = grad.reshape(-1, 4)[pix]
    rz, rd = blend_backward(hp, hz, hd, colors, prm, gs)
    sc = blend_backward_scale(hp, hz, hd, colors, prm, gs)
    _check(ref, sel(rgba, (4,)), (rz, rd), (sel(gz, (K,)), sel(gd, (K,))), sc)


def test_blend_full_size_dense(dmr):
    # every pixel of every image of hetero16_256 (16 x 256 x 256 x 10 slots),
    # and every pixel of the soups32_512 image with the largest soup
    # (512 x 512 x 50 slots), each blended at full size in one launch
    prm = PARAMS["sharp"]
    for name in ("hetero16_256", "soups32_512"):
        w = make_workload(name)
        say(f"[gpu] blend {name} dense")
        g = GpuCase.from_workload(w)
        p2f, zbuf, _, dists = g.forward()
        colors = face_colors(w)
        grad = blend_upstream_grads(w)
        rgba, gz, gd = _blend_gpu(dmr, p2f, zbuf, dists, to_dev(colors), prm, to_dev(grad))
        imgs = range(w.N) if name == "hetero16_256" else [int(np.diff(w.offsets).argmax())]
        for n in imgs:
            hp, hz, hd = p2f[n].cpu().numpy(), zbuf[n].cpu().numpy(), dists[n].cpu().numpy()
            gs = grad[n]
            ref = blend_forward(hp, hz, hd, colors, prm)
            rz, rd = blend_backward(hp, hz, hd, colors, prm, gs)
            sc = blend_backward_scale(hp, hz, hd, colors, prm, gs)
            _check(ref, rgba[n].cpu().numpy(), (rz, rd), (gz[n].cpu().numpy(), gd[n].cpu().numpy()), sc)
            assert (hp >= 0).any()


@pytest.mark.parametrize("K", [1, 20, 64])
def test_blend_edge_slots(dmr, K):
    # empty pixels, out-of-range face indices (empty slots), ties; K = 20 and
    # 64 take several slot chunks, the last one partial for K = 20; P = 300
    # leaves a partial block of pixels
    rng = np.random.default_rng(3 + K)
    P, F = 300, 50
    p2f = rng.integers(-1, F + 5, (P, K)).astype(np.int64)
    p2f[:40] = -1
    zbuf = rng.uniform(1.0, 3.0, (P, K)).astype(np.float32)
    zbuf[40:60] = 2.0
    dists = rng.normal(0, 5e-4, (P, K)).astype(np.float32)
    colors = rng.random((F, 3), dtype=np.float32)
    grad = rng.standard_normal((P, 4), dtype=np.float32)
    prm = PARAMS["soft_near_bg"]
    say(f"[gpu] blend edge slots K={K}")
    rgba, gz, gd = _blend_gpu(dmr, to_dev(p2f), to_dev(zbuf), to_dev(dists), to_dev(colors), prm, to_dev(grad))
    p2f_ref = np.where(p2f < F, p2f, -1)
    ref = blend_forward(p2f_ref, zbuf, dists, colors, prm)
    rz, rd = blend_backward(p2f_ref, zbuf, dists, colors, prm, grad)
    sc = blend_backward_scale(p2f_ref, zbuf, dists, colors, prm, grad)
    _check(ref, rgba.cpu().numpy(), (rz, rd), (gz.cpu().numpy(), gd.cpu().numpy()), sc)
    assert (rgba[:40].cpu().numpy() == np.array([0.2, 0.4, 0.9, 0.0], np.float32)).all()

"""Point-cloud rasterization on the GPU (through the C ABI) against its
oracle (oracle/points.py, binary32 in the same operation order): idx, zbuf
and dists must match bit for bit, padding included; grad_points within 1e-5
relative L2 (float32 atomics reorder the sums)."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, require_gpu, say, to_dev
from oracle.points import rasterize_points, rasterize_points_backward
from parity import point_oracle_band, rel_l2
from workloads import make_point_workload, point_upstream_grads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dmr():
    return require_gpu()


def _gpu(dmr, pts, off, H, W, K, radius, ws_bytes=None):
    p, o = to_dev(np.asarray(pts, np.float32)), to_dev(np.asarray(off, np.int64))
    N = len(off) - 1
    shape = (N, H, W, K)
    idx = torch.empty(shape, dtype=torch.int64, device=DEV)
    zb = torch.empty(shape, dtype=torch.float32, device=DEV)
    ds = torch.empty(shape, dtype=torch.float32, device=DEV)
    if ws_bytes is None:
        ws_bytes = dmr.dmr_points_workspace_size_hint(N, p.shape[0], H, W, K, radius)
    ws = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device=DEV)
    dmr.rasterize_points_fwd(p, o, H, W, K, radius, idx, zb, ds, ws)
    torch.cuda.synchronize()
    return (idx, zb, ds), (p, o), ws


def _exact(got, ref):
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g.cpu().numpy(), r)


@pytest.mark.parametrize("name", ["points_small", "points_soup"])
def test_points_full_image(dmr, name):
    w = make_point_workload(name)
    say(f"[gpu] points full image {name} N={w.N} P={w.P} {w.H}x{w.W} K={w.K} r={w.radius}")
    out, (p, o), ws = _gpu(dmr, w.points, w.offsets, w.H, w.W, w.K, w.radius)
    ref = rasterize_points(w.points, w.offsets, w.H, w.W, w.K, w.radius)
    _exact(out, ref)
    assert (ref[0] >= 0).sum() > 1000
    st = dmr.dmr_workspace_stats(ws)
    assert st["overflow_bins"] == 0
    g = point_upstream_grads(w)
    gp = torch.empty_like(p)
    dmr.rasterize_points_bwd(p, o, w.H, w.W, w.K, out[0], to_dev(g["zbuf"]), to_dev(g["dists"]), gp)
    refg = rasterize_points_backward(w.points, w.offsets, w.H, w.W, w.K, ref[0], g["zbuf"], g["dists"])
    err = rel_l2(gp.cpu().numpy(), refg)
    say(f"  backward rel L2 = {err:.2e}")
    assert np.linalg.norm(refg) > 0 and err <= 1e-5


def test_points_full_size_sampled(dmr):
    w = make_point_workload("points16_256")
    rng = np.random.default_rng(12)
    pix = np.unique(rng.integers(0, w.pixels, 4000))
    say(f"[gpu] points full size points16_256 P={w.P}, {len(pix)} sampled pixels")
    out, (p, o), ws = _gpu(dmr, w.points, w.offsets, w.H, w.W, w.K, w.radius)
    st = dmr.dmr_workspace_stats(ws)
    say(f"  stats {st}")
    assert st["overflow_bins"] == 0
    ref = rasterize_points(w.points, w.offsets, w.H, w.W, w.K, w.radius, pixels=pix)
    idx_t = torch.from_numpy(pix).to(DEV)
    for g, r in zip(out, ref):
        got = g.reshape(-1, w.K).index_select(0, idx_t).cpu().numpy()
        np.testing.assert_array_equal(got, r)
    # whole image: filled slots form a prefix, keys ascend
    idx, zb = out[0], out[1]
    filled = idx >= 0
    assert bool((filled[..., 1:] <= filled[..., :-1]).all())
    z = torch.where(filled, zb, torch.full_like(zb, float("inf")))
    assert bool((z[..., 1:] >= z[..., :-1]).all())
    assert filled.float().mean().item() > 0.05
    # backward: upstream gradients on the sampled pixels only
    g = point_upstream_grads(w)
    shape = (w.N, w.H, w.W, w.K)
    dense = {}
    for k in ("zbuf", "dists"):
        full = torch.zeros(shape, dtype=torch.float32, device=DEV)
        full.view(-1, w.K).index_copy_(0, idx_t, to_dev(g[k].reshape(-1, w.K)[pix]))
        dense[k] = full
    gp = torch.empty_like(p)
    dmr.rasterize_points_bwd(p, o, w.H, w.W, w.K, idx, dense["zbuf"], dense["dists"], gp)
    refg = rasterize_points_backward(w.points, w.offsets, w.H, w.W, w.K, ref[0], g["zbuf"].reshape(-1, w.K)[pix],
                                     g["dists"].reshape(-1, w.K)[pix], pixels=pix)
    assert rel_l2(gp.cpu().numpy(), refg) <= 1e-5


def test_points_full_size_dense_largest_cloud(dmr):
    """points16_256 in the bench's launch configuration: every pixel of the
    image of its largest cloud, bit for bit against the oracle (16 bands of
    16 rows); then the backward pass with N(0,1) upstream gradients on every
    slot of that image (zero elsewhere) against the oracle's sum."""
    w = make_point_workload("points16_256")
    n = int(np.argmax(np.diff(w.offsets)))
    say(f"[gpu] points dense whole image {n} of points16_256 ({int(np.diff(w.offsets)[n])} points)")
    out, (p, o), _ = _gpu(dmr, w.points, w.offsets, w.H, w.W, w.K, w.radius)
    got = [t[n].cpu().numpy().reshape(w.H * w.W, w.K) for t in out]
    pts_np = np.asarray(w.points, np.float32).reshape(-1, 3)
    filled = 0
    ref_idx = []
    for r0 in range(0, w.H, 16):
        r1 = min(w.H, r0 + 16)
        ref = point_oracle_band(rasterize_points, w, n, r0, r1, pts_np)
        rows = slice(r0 * w.W, r1 * w.W)
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g[rows], r)
        filled += int((ref[0] >= 0).sum())
        ref_idx.append(ref[0])
    say(f"  {filled} filled slots, all equal")
    assert filled > 0
    rng = np.random.Generator(np.random.PCG64(77 + n))
    gz = rng.standard_normal((w.H * w.W, w.K), dtype=np.float32)
    gd = rng.standard_normal((w.H * w.W, w.K), dtype=np.float32)
    shape = (w.N, w.H, w.W, w.K)
    dz = torch.zeros(shape, dtype=torch.float32, device=DEV)
    dd = torch.zeros(shape, dtype=torch.float32, device=DEV)
    dz[n] = to_dev(gz.reshape(w.H, w.W, w.K))
    dd[n] = to_dev(gd.reshape(w.H, w.W, w.K))
    gp = torch.empty_like(p)
    dmr.rasterize_points_bwd(p, o, w.H, w.W, w.K, out[0], dz, dd, gp)
    pix = n * w.H * w.W + np.arange(w.H * w.W, dtype=np.int64)
    refg = rasterize_points_backward(w.points, w.offsets, w.H, w.W, w.K, np.concatenate(ref_idx), gz, gd, pixels=pix)
    err = rel_l2(gp.cpu().numpy(), refg)
    say(f"  backward rel L2 = {err:.2e}")
    assert np.linalg.norm(refg) > 0
    assert err <= 1e-5


def test_points_small_workspace_is_exact(dmr):
    w = make_point_workload("points_soup")
    say("[gpu] points with a minimal workspace (every bin list overflows)")
    ws_min = dmr.dmr_points_workspace_min_size(w.N, w.P, w.H, w.W)
    out, _, ws = _gpu(dmr, w.points, w.offsets, w.H, w.W, w.K, w.radius, ws_bytes=ws_min)
    assert dmr.dmr_workspace_stats(ws)["overflow_bins"] > 0
    _exact(out, rasterize_points(w.points, w.offsets, w.H, w.W, w.K, w.radius))


EDGE_CASES = ["k1", "k64", "radius0", "empty_clouds", "offscreen", "ragged", "dense_bin"]


@pytest.mark.parametrize("case", EDGE_CASES)
def test_points_edge_cases(dmr, case):
    rng = np.random.default_rng(EDGE_CASES.index(case))
    H, W, K, radius = 37, 29, 4, 0.05
    pts = np.concatenate([rng.uniform(-1, 1, (600, 2)), rng.uniform(0.5, 2, (600, 1))], 1)
    off = [0, 300, 600]
    if case == "k1":
        K = 1
    elif case == "k64":
        K, radius = 64, 0.15
    elif case == "radius0":
        radius = 0.0
    elif case == "empty_clouds":
        off = [0, 0, 600, 600]
    elif case == "offscreen":
        pts[:, :2] *= 3.0
    elif case == "ragged":
        H, W = 1, 53
    elif case == "dense_bin":
        # 5000 points within one 16x16 bin: a list longer than the sort holds
        pts = np.concatenate([rng.uniform(-0.95, -0.9, (5000, 2)), rng.uniform(0.5, 2, (5000, 1))], 1)
        off, H, W, K, radius = [0, 5000], 64, 64, 8, 0.02
    pts = pts.astype(np.float32)
    say(f"[gpu] points edge case {case}")
    out, _, _ = _gpu(dmr, pts, off, H, W, K, radius)
    ref = rasterize_points(pts, off, H, W, K, radius)
    _exact(out, ref)
    if case == "radius0":
        assert (ref[0] == -1).all()


def test_points_autograd(dmr):
    w = make_point_workload("points_small")
    p = to_dev(w.points).requires_grad_(True)
    idx, zb, ds = dmr.rasterize_points(p, to_dev(w.offsets), (w.H, w.W), w.K, w.radius)
    g = point_upstream_grads(w)
    ((zb * to_dev(g["zbuf"])).sum() + (ds * to_dev(g["dists"])).sum()).backward()
    ref = rasterize_points(w.points, w.offsets, w.H, w.W, w.K, w.radius)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref[0])
    refg = rasterize_points_backward(w.points, w.offsets, w.H, w.W, w.K, ref[0], g["zbuf"], g["dists"])
    assert rel_l2(p.grad.cpu().numpy(), refg) <= 1e-5


@pytest.mark.parametrize("scale", [1e-10, 1e-8, 1e-6, 1e6])
def test_points_backward_gradient_scales(dmr, scale):
    """The point backward shares the per-tile fixed-point table: its accuracy
    must not depend on the scale of the upstream gradients (all coordinates,
    and the depth coordinates alone)."""
    w = make_point_workload("points_small")
    say(f"[gpu] points backward with upstream gradients scaled by {scale}")
    out, (p, o), ws = _gpu(dmr, w.points, w.offsets, w.H, w.W, w.K, w.radius)
    g = {k: (a * np.float32(scale)).astype(np.float32) for k, a in point_upstream_grads(w).items()}
    gp = torch.empty_like(p)
    dmr.rasterize_points_bwd(p, o, w.H, w.W, w.K, out[0], to_dev(g["zbuf"]), to_dev(g["dists"]), gp)
    refg = rasterize_points_backward(w.points, w.offsets, w.H, w.W, w.K, out[0].cpu().numpy(), g["zbuf"],
                                     g["dists"])
    got = gp.cpu().numpy()
    err, err_z = rel_l2(got, refg), rel_l2(got[:, 2], refg[:, 2])
    say(f"  rel L2 = {err:.2e}, depth coordinates {err_z:.2e}")
    assert np.linalg.norm(refg[:, 2]) > 0
    assert err <= 1e-5 and err_z <= 1e-5, (err, err_z)

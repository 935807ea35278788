"""Rasterizer settings on the GPU (through the C ABI) against the oracle with
the same settings: perspective-correct barycentrics, back-face culling and
unclipped barycentrics, alone and combined.

The bar is that of the default path: pix_to_face bit for bit except at
near-threshold pixels (with the oracle's excuse rule under the same
settings), zbuf/bary/dists within 1e-5 absolute, padding exactly -1,
grad_verts within 1e-4 relative L2 (with and without the forward's
workspace)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, GpuCase, dense_region_check, host, require_gpu, rows, say, to_dev
from parity import assert_forward_parity, compare_forward, oracle_excuse, rel_l2
from workloads import make_workload, masked_upstream_grads, sample_pixels, upstream_grads

pytestmark = pytest.mark.gpu

P, C, U = oracle.PERSPECTIVE, oracle.CULL_BACKFACES, oracle.UNCLIPPED_BARY
SETTINGS = {"persp": P, "cull": C, "unclipped": U, "persp_unclipped": P | U, "all": P | C | U}


@pytest.fixture(scope="module")
def dmr():
    d = require_gpu()
    assert (d.DMR_RASTER_PERSPECTIVE_CORRECT, d.DMR_RASTER_CULL_BACKFACES, d.DMR_RASTER_UNCLIPPED_BARY) == (P, C, U)
    return d


def _dense_grads(w):
    gr = upstream_grads(w)
    return gr, [None if gr[k] is None else to_dev(gr[k]) for k in ("zbuf", "bary", "dists")]


@pytest.mark.parametrize("sname", list(SETTINGS))
@pytest.mark.parametrize("name", ["spheres8_137", "small_hetero", "small_soups"])
def test_settings_full_image(dmr, name, sname):
    settings = SETTINGS[sname]
    w = make_workload(name)
    say(f"[gpu] settings {sname} forward+backward full image {name} N={w.N} F={w.F} {w.H}x{w.W} K={w.K}")
    g = GpuCase.from_workload(w)
    out = g.forward(settings=settings)
    got = host(out)
    ref = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, settings=settings)
    rep = compare_forward(ref, got, w.K, excuse=oracle_excuse(oracle, w.verts, w.faces, w.offsets, w.H, w.W, w.blur,
                                                               settings=settings))
    say(f"  filled={rep['filled_slots']} excused={len(rep['excused'])} "
        f"err z/b/d={rep['max_err_zbuf']:.2e}/{rep['max_err_bary']:.2e}/{rep['max_err_dists']:.2e}")
    assert_forward_parity(rep)
    assert rep["filled_slots"] > 0
    assert np.array_equal(got[0], ref[0])
    gr, (dz, db, dd) = _dense_grads(w)
    refg = oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, ref[0], gr["zbuf"], gr["bary"],
                           gr["dists"], settings=settings)
    assert np.linalg.norm(refg) > 0
    for reuse in (True, False):
        gv = g.backward(out[0], dz, db, dd, reuse=reuse).cpu().numpy()
        err = rel_l2(gv, refg)
        say(f"  backward reuse={reuse} rel L2 = {err:.2e}")
        assert err <= 1e-4


def test_settings_change_the_outputs(dmr):
    # each setting changes what it should on spheres8_137, and nothing else
    w = make_workload("spheres8_137")
    g = GpuCase.from_workload(w)
    base = host(g.forward())
    persp = host(g.forward(settings=P))
    unclipped = host(g.forward(settings=U))
    culled = host(g.forward(settings=C))
    filled = base[0] >= 0
    assert not np.array_equal(base[1][filled], persp[1][filled])
    # where the K slots hold every candidate, the sets agree (the order may not)
    room = base[0][..., -1] < 0
    assert room.mean() > 0.5
    np.testing.assert_array_equal(np.sort(base[0][room], -1), np.sort(persp[0][room], -1))
    for k in (0, 1, 3):
        np.testing.assert_array_equal(base[k], unclipped[k])
    assert (unclipped[2] < 0).any() and not (unclipped[2][filled] < 0).all()
    assert (culled[0] >= 0).sum() < filled.sum()
    # culling only removes candidates
    for a, b in zip(culled[0][room], base[0][room]):
        assert set(a[a >= 0].tolist()) <= set(b[b >= 0].tolist())


@pytest.mark.parametrize("sname", ["persp", "all"])
def test_settings_full_size_sampled(dmr, sname):
    settings = SETTINGS[sname]
    w = make_workload("hetero16_256")
    pix = sample_pixels(w, 2000, seed=11)
    say(f"[gpu] settings {sname} full size hetero16_256, {len(pix)} sampled pixels")
    g = GpuCase.from_workload(w)
    out = g.forward(settings=settings)
    got = rows(out, pix, w.K)
    ref = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, pixels=pix, settings=settings)
    rep = compare_forward(ref, got, w.K, excuse=oracle_excuse(oracle, w.verts, w.faces, w.offsets, w.H, w.W, w.blur,
                                                               pixel_ids=pix, settings=settings))
    say(f"  filled={rep['filled_slots']} excused={len(rep['excused'])}")
    assert_forward_parity(rep, max_excused_frac=max(1e-4, 1.0 / len(pix)))
    sg = masked_upstream_grads(w, pix)
    shape = (w.N, w.H, w.W, w.K)
    idx = torch.from_numpy(pix).to(DEV)
    dense = {}
    for key in ("zbuf", "bary", "dists"):
        if sg[key] is None:
            dense[key] = None
            continue
        full = torch.zeros(shape + ((3,) if key == "bary" else ()), dtype=torch.float32, device=DEV)
        full.view((-1, w.K) + ((3,) if key == "bary" else ())).index_copy_(0, idx, to_dev(sg[key]))
        dense[key] = full
    gv = g.backward(out[0], dense["zbuf"], dense["bary"], dense["dists"]).cpu().numpy()
    refg = oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, ref[0], sg["zbuf"], sg["bary"],
                           sg["dists"], pixels=pix, settings=settings)
    err = rel_l2(gv, refg)
    say(f"  backward rel L2 = {err:.2e}")
    assert err <= 1e-4


@pytest.mark.parametrize("sname", ["persp", "cull", "all"])
def test_settings_dense_largest_mesh_hetero(dmr, sname):
    """hetero16_256 in the benchmark's launch configuration under a setting:
    every pixel of the image of its largest mesh (65,536 pixels, K = 10),
    forward and backward, against the oracle with the same setting."""
    settings = SETTINGS[sname]
    w = make_workload("hetero16_256")
    n = int(np.argmax(np.diff(w.offsets)))
    say(f"[gpu] settings {sname}: dense whole image {n} of hetero16_256 ({int(np.diff(w.offsets)[n])} faces)")
    g = GpuCase.from_workload(w)
    out = g.forward(settings=settings)
    dense_region_check(w, g, out, n, [(i0, min(w.H, i0 + 16)) for i0 in range(0, w.H, 16)], settings=settings)


def test_autograd_wrapper_settings(dmr):
    w = make_workload("small_hetero")
    v = to_dev(w.verts).requires_grad_(True)
    f, o = to_dev(w.faces), to_dev(w.offsets)
    p2f, zbuf, bary, dists = dmr.rasterize_meshes(v, f, o, (w.H, w.W), w.K, w.blur, perspective_correct=True,
                                                  cull_backfaces=True, clip_barycentric_coords=False)
    ref = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, settings=P | C | U)
    np.testing.assert_array_equal(p2f.cpu().numpy(), ref[0])
    gr = upstream_grads(w)
    loss = sum((t * to_dev(gr[k])).sum() for t, k in ((zbuf, "zbuf"), (bary, "bary"), (dists, "dists"))
               if gr[k] is not None)
    loss.backward()
    refg = oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, ref[0], gr["zbuf"], gr["bary"],
                           gr["dists"], settings=P | C | U)
    assert rel_l2(v.grad.cpu().numpy(), refg) <= 1e-4

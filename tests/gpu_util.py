"""Helpers for the GPU tests: move seeded numpy inputs to the device, call the
C-ABI entry points through the Python binding, bring results back."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import assert_forward_parity, compare_forward, oracle_excuse, oracle_region, rel_l2

DEV = torch.device("cuda:0")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import differentiable_mesh_rasterization_amd as dmr

    dmr.lib()  # raises if the HIP library is not built: no silent fallback
    return dmr


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


class GpuCase:
    """Device copies of one workload's inputs."""

    def __init__(self, verts, faces, offsets, H, W, K, blur):
        self.verts = to_dev(np.asarray(verts, np.float32).reshape(-1, 3))
        self.faces = to_dev(np.asarray(faces, np.int64).reshape(-1, 3))
        self.offsets = to_dev(np.asarray(offsets, np.int64))
        self.H, self.W, self.K, self.blur = int(H), int(W), int(K), float(blur)
        self.N = self.offsets.shape[0] - 1

    @classmethod
    def from_workload(cls, w):
        return cls(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur)

    def forward(self, ws_bytes=None, out=None, settings=None):
        """Forward pass (rasterize_meshes_fwd, or rasterize_meshes_fwd_ex
        with `settings`); the settings are kept for backward()."""
        import differentiable_mesh_rasterization_amd as dmr

        N, H, W, K = self.N, self.H, self.W, self.K
        if out is None:
            out = (torch.empty((N, H, W, K), dtype=torch.int64, device=DEV),
                   torch.empty((N, H, W, K), dtype=torch.float32, device=DEV),
                   torch.empty((N, H, W, K, 3), dtype=torch.float32, device=DEV),
                   torch.empty((N, H, W, K), dtype=torch.float32, device=DEV))
        if ws_bytes is None:
            ws_bytes = dmr.dmr_workspace_size_hint(N, self.faces.shape[0], H, W, K, self.blur)
        ws = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device=DEV)
        if settings is None:
            dmr.rasterize_meshes_fwd(self.verts, self.faces, self.offsets, H, W, K, self.blur, *out, ws)
        else:
            dmr.rasterize_meshes_fwd_ex(self.verts, self.faces, self.offsets, H, W, K, self.blur, *out, ws,
                                        settings)
        torch.cuda.synchronize()
        self.ws = ws
        self.settings = settings or 0
        return out

    def backward(self, p2f, gz=None, gb=None, gd=None, reuse=True):
        """Backward pass; with reuse=True it takes the workspace of the last
        forward() call (same inputs), otherwise none (face data recomputed)."""
        import differentiable_mesh_rasterization_amd as dmr

        gv = torch.empty_like(self.verts)
        ws = self.ws if reuse else None
        dmr.rasterize_meshes_bwd(self.verts, self.faces, self.offsets, self.H, self.W, self.K, self.blur, p2f,
                                 gz, gb, gd, gv, ws, reuse_forward_workspace=reuse,
                                 settings=getattr(self, "settings", 0))
        torch.cuda.synchronize()
        return gv

    def stats(self):
        import differentiable_mesh_rasterization_amd as dmr

        return dmr.dmr_workspace_stats(self.ws)


def host(out):
    return tuple(t.cpu().numpy() for t in out)


def rows(out, pixel_ids, K):
    """Selected pixel rows of device outputs, copied to the host."""
    idx = torch.from_numpy(np.asarray(pixel_ids, np.int64)).to(DEV)
    res = []
    for t in out:
        flat = t.reshape((-1, K) + tuple(t.shape[4:]))
        res.append(flat.index_select(0, idx).cpu().numpy())
    return tuple(res)


def say(*a):
    print(*a, flush=True)


def dense_region_check(w, g, out, n, bands, settings=0):
    """Every pixel of the given row bands [(i0, i1)] of image n, full width:
    the forward outputs against the oracle, and the backward pass with N(0,1)
    upstream gradients on those pixels only (zero elsewhere) against the
    oracle's sum over them. The oracle runs band by band on the faces that
    can reach the band (parity.oracle_region), under the rasterizer settings
    `settings`: those `out` was computed with (g.backward applies the
    settings of g's last forward call)."""
    rng = np.random.Generator(np.random.PCG64(4242 + n))
    shape = (w.N, w.H, w.W, w.K)
    dense = {k: (torch.zeros(shape + ((3,) if k == "bary" else ()), dtype=torch.float32, device=DEV)
                 if k in w.grads else None) for k in ("zbuf", "bary", "dists")}
    reports, ref_gv = [], np.zeros((w.V, 3))
    for i0, i1 in bands:
        npx = (i1 - i0) * w.W
        gr = {k: (rng.standard_normal((npx, w.K) + ((3,) if k == "bary" else ()), dtype=np.float32)
                  if k in w.grads else None) for k in ("zbuf", "bary", "dists")}
        pix, ref, gv = oracle_region(oracle, w.verts, w.faces, w.offsets, n, w.H, w.W, w.K, w.blur, i0, i1, 0, w.W,
                                     grads=(gr["zbuf"], gr["bary"], gr["dists"]), settings=settings)
        ref_gv += gv
        got = rows(out, pix, w.K)
        reports.append(compare_forward(ref, got, w.K, excuse=oracle_excuse(oracle, w.verts, w.faces, w.offsets, w.H,
                                                                           w.W, w.blur, pixel_ids=pix,
                                                                           settings=settings)))
        for k, t in dense.items():
            if t is not None:
                t[n, i0:i1] = to_dev(gr[k].reshape((i1 - i0, w.W, w.K) + t.shape[4:]))
    rep = {"pixels": sum(r["pixels"] for r in reports),
           "excused": sum((r["excused"] for r in reports), []), "unexcused": sum((r["unexcused"] for r in reports), []),
           "max_err_zbuf": max(r["max_err_zbuf"] for r in reports),
           "max_err_bary": max(r["max_err_bary"] for r in reports),
           "max_err_dists": max(r["max_err_dists"] for r in reports),
           "padding_ok": all(r["padding_ok"] for r in reports), "values_ok": all(r["values_ok"] for r in reports),
           "filled_slots": sum(r["filled_slots"] for r in reports)}
    say(f"  {rep['pixels']} pixels, filled={rep['filled_slots']} excused={len(rep['excused'])} "
        f"err z/b/d={rep['max_err_zbuf']:.2e}/{rep['max_err_bary']:.2e}/{rep['max_err_dists']:.2e}")
    assert rep["filled_slots"] > 0
    assert_forward_parity(rep, max_excused_frac=1e-4)
    gv = g.backward(out[0], dense["zbuf"], dense["bary"], dense["dists"]).cpu().numpy()
    err, err_z = rel_l2(gv, ref_gv), rel_l2(gv[:, 2], ref_gv[:, 2])
    say(f"  backward rel L2 = {err:.2e}, depth coordinates {err_z:.2e}")
    assert np.linalg.norm(ref_gv) > 0
    assert err <= 1e-4 and err_z <= 1e-4

"""The allocation-free forward entry point (rasterize_meshes_fwd_noalloc,
whose workspace is the library's per-device scratch array) against the
ordinary forward entry point with a caller-allocated workspace: outputs bit
for bit identical, over two calls in a row with the second on a smaller
input (the array keeps the first call's contents), and sizes beyond the
array rejected before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV, GpuCase, host, require_gpu, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dmr():
    return require_gpu()


def _noalloc(dmr, g):
    out = (torch.empty((g.N, g.H, g.W, g.K), dtype=torch.int64, device=DEV),
           torch.empty((g.N, g.H, g.W, g.K), dtype=torch.float32, device=DEV),
           torch.empty((g.N, g.H, g.W, g.K, 3), dtype=torch.float32, device=DEV),
           torch.empty((g.N, g.H, g.W, g.K), dtype=torch.float32, device=DEV))
    dmr.rasterize_meshes_fwd_noalloc(g.verts, g.faces, g.offsets, g.H, g.W, g.K, g.blur, *out)
    torch.cuda.synchronize()
    return host(out)


def test_noalloc_matches_workspace_entry_point(dmr):
    for name in ("hetero16_256", "small_hetero"):   # the second call is smaller
        w = make_workload(name)
        say(f"[gpu] allocation-free forward on {name} N={w.N} F={w.F} {w.H}x{w.W} K={w.K}")
        g = GpuCase.from_workload(w)
        ref = host(g.forward())
        got = _noalloc(dmr, g)
        for a, b in zip(ref, got):
            assert a.shape == b.shape
            assert np.array_equal(a, b)
        assert (ref[0] >= 0).sum() > 1000


def test_noalloc_backward_after_noalloc_forward(dmr):
    """The backward pass without the forward's workspace allocates nothing
    either; it equals the one that reuses a caller-allocated workspace."""
    from parity import rel_l2
    from workloads import upstream_grads
    from gpu_util import to_dev

    w = make_workload("small_soups")
    say("[gpu] allocation-free forward, then backward without a workspace")
    g = GpuCase.from_workload(w)
    ref = g.forward()
    got = _noalloc(dmr, g)
    assert np.array_equal(got[0], ref[0].cpu().numpy())
    gr = upstream_grads(w)
    args = (to_dev(got[0]), to_dev(gr["zbuf"]), to_dev(gr["bary"]), to_dev(gr["dists"]))
    a = g.backward(*args, reuse=True).cpu().numpy()
    b = g.backward(*args, reuse=False).cpu().numpy()
    assert rel_l2(b, a) <= 1e-6


def test_noalloc_rejects_sizes_beyond_the_array(dmr):
    """Face records and bin tables beyond the array: DMR_ERROR_UNSUPPORTED,
    decided on the host before any launch (the pointers are never read)."""
    L = dmr.lib()
    F = dmr.DMR_NOALLOC_SCRATCH_BYTES // 64 + 1   # 64-byte records alone exceed it
    assert dmr.dmr_workspace_min_size(1, F, 64, 64) > dmr.DMR_NOALLOC_SCRATCH_BYTES
    # real buffers of the stated sizes, so that nothing could be read out
    # of bounds even if the call went ahead
    verts = torch.zeros((3, 3), dtype=torch.float32, device=DEV)
    faces = torch.zeros((F, 3), dtype=torch.int64, device=DEV)
    offsets = torch.tensor([0, F], dtype=torch.int64, device=DEV)
    out = [torch.empty((1, 64, 64, 1) + t, dtype=d, device=DEV)
           for t, d in (((), torch.int64), ((), torch.float32), ((3,), torch.float32), ((), torch.float32))]

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr())

    rc = L.rasterize_meshes_fwd_noalloc(ptr(verts), 3, ptr(faces), F, ptr(offsets), 1, 64, 64, 1, 0.0,
                                        *[ptr(t) for t in out], None)
    torch.cuda.synchronize()
    assert rc == 4   # DMR_ERROR_UNSUPPORTED
    assert dmr.dmr_workspace_min_size(1, 1000, 64, 64) <= dmr.DMR_NOALLOC_SCRATCH_BYTES

#!/usr/bin/env python3
"""Benchmark: forward+backward K-nearest-face mesh rasterization on one MI355X.

One step = rasterize_meshes_fwd + rasterize_meshes_bwd (every stage of the
path: face setup, bin count, scan, bin fill, bin sort, fine raster, gradient
zeroing, backward) over one batch of seeded synthetic meshes already
resident in HBM. The headline workload is a heterogeneous batch of 16
icospheres (levels 3-6, 1280-81920 triangles each) at 256x256, K = 10,
blur_radius = 1e-4.

Prints one JSON line:
  value / ms_per_step   whole-step throughput of the headline workload
                        (Mpixel*K slots per second);
  roofline              the dominant kernel against HBM bandwidth, timed with
                        HIP events on the stream it runs on inside the timed
                        region;
  valu                  the step's algorithmic fp32 flops against the fp32
                        vector peak (packed, and the unpacked peak the
                        kernels can reach without packed instructions);
  configs               every workload of the benchmark suite (a 64x64
                        sphere, 8 spheres at 137x137, the headline batch, a
                        1M-triangle soup at 1024x1024, 32 soups at 512x512
                        with K = 50), each forward only and forward+backward,
                        with its HBM and fp32-VALU fractions and kernel times;
  cpu_baseline          the CPU oracle timed on a bounded pixel sample of the
                        headline workload on this host, and
  parity                the GPU outputs compared with the oracle's on sampled
                        pixels of every workload (the headline one on the
                        cpu_baseline sample).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload hetero16_256]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
VALU_PEAK_TFLOPS = 157.3     # MI355X fp32 vector (packed), TFLOP/s
# The kernels are built without packed fp32 instructions, so one lane
# retires one fp32 operation per instruction: half the packed peak.
VALU_UNPACKED_TFLOPS = 78.6

METRIC = "forward+backward Mpixels*K/s at 1 MI355X; % of fp32-VALU/HBM roofline"
SUITE = ("sphere64", "spheres8_137", "hetero16_256", "soup1m_1024", "soups32_512")

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move and compute, per launch)
# ---------------------------------------------------------------------------

def grad_bytes_per_filled_slot(grads) -> int:
    return (4 if "zbuf" in grads else 0) + (12 if "bary" in grads else 0) + (4 if "dists" in grads else 0)


def algorithmic_bytes(w, filled_slots):
    """Forward: 28 B per slot written (index 8, depth 4, barycentrics 12,
    distance 4; padding included) + 24 B per face + 12 B per vertex read.
    Backward: 8 B per slot (the face index) + the supplied upstream
    gradients per filled slot + 24 B per face + 12 B per vertex read + 12 B
    per vertex written."""
    fwd = 28 * w.slots + 24 * w.F + 12 * w.V
    bwd = 8 * w.slots + grad_bytes_per_filled_slot(w.grads) * filled_slots + 24 * w.F + 24 * w.V
    return {"fine_raster": fwd, "backward_slots": bwd, "fwd_total": fwd, "bwd_total": bwd}


def pair_counts(w, sample_pairs: int = 3_000_000, seed: int = 5):
    """(P_bbox, P_acc): pixel centres inside a live face's box grown by the
    blur radius, counted exactly over all faces, and the (pixel, face) pairs
    that are candidates (inside, or squared distance below the blur radius,
    with a positive depth), counted in binary64 on a random subset of faces
    holding about `sample_pairs` box pairs and scaled to all faces (exact
    when the subset is every face). A measure of work, not a result."""
    import numpy as np

    v = w.verts.astype(np.float64)
    tri = v[w.faces]                                   # [F, 3, 3]
    x, y, z = tri[..., 0], tri[..., 1], tri[..., 2]
    A = (x[:, 1] - x[:, 0]) * (y[:, 2] - y[:, 0]) - (y[:, 1] - y[:, 0]) * (x[:, 2] - x[:, 0])
    live = (A != 0) & (z.max(axis=1) > 0)
    r = np.sqrt(w.blur)
    j0 = np.maximum(np.ceil(((x.min(1) - r + 1.0) * w.W - 1.0) / 2.0), 0)
    j1 = np.minimum(np.floor(((x.max(1) + r + 1.0) * w.W - 1.0) / 2.0), w.W - 1)
    i0 = np.maximum(np.ceil(((y.min(1) - r + 1.0) * w.H - 1.0) / 2.0), 0)
    i1 = np.minimum(np.floor(((y.max(1) + r + 1.0) * w.H - 1.0) / 2.0), w.H - 1)
    nbox = np.where(live, np.maximum(j1 - j0 + 1, 0) * np.maximum(i1 - i0 + 1, 0), 0).astype(np.int64)
    p_bbox = int(nbox.sum())
    if p_bbox == 0:
        return 0, 0
    rng = np.random.Generator(np.random.PCG64(seed))
    frac = min(1.0, sample_pairs / p_bbox)
    pick = np.nonzero((nbox > 0) & (rng.random(w.F) < frac))[0]
    counts = nbox[pick]
    fid = np.repeat(pick, counts)
    k = np.arange(len(fid)) - np.repeat(np.cumsum(counts) - counts, counts)
    ncol = np.repeat((j1 - j0 + 1)[pick].astype(np.int64), counts)
    px = (2.0 * (j0[fid] + k % ncol) + 1.0) / w.W - 1.0
    py = (2.0 * (i0[fid] + k // ncol) + 1.0) / w.H - 1.0
    X, Y, Z = x[fid], y[fid], z[fid]
    dx, dy = X - px[:, None], Y - py[:, None]
    wk = np.stack([dx[:, 1] * dy[:, 2] - dy[:, 1] * dx[:, 2], dx[:, 2] * dy[:, 0] - dy[:, 2] * dx[:, 0],
                   dx[:, 0] * dy[:, 1] - dy[:, 0] * dx[:, 1]], 1) / A[fid][:, None]
    inside = (wk > 0).all(axis=1)
    d2 = np.full(len(fid), np.inf)
    for e in range(3):
        a, b = e, (e + 1) % 3
        ux, uy = X[:, b] - X[:, a], Y[:, b] - Y[:, a]
        qx, qy = px - X[:, a], py - Y[:, a]
        t = np.clip((qx * ux + qy * uy) / (ux * ux + uy * uy), 0.0, 1.0)
        d2 = np.minimum(d2, (qx - t * ux) ** 2 + (qy - t * uy) ** 2)
    c = np.clip(wk, 0.0, 1.0)
    zz = (c * Z).sum(1) / c.sum(1)
    acc = (inside | (d2 < w.blur)) & (zz > 0)
    sampled_bbox = int(counts.sum())
    p_acc = int(round(acc.sum() * (p_bbox / sampled_bbox))) if sampled_bbox else 0
    return p_bbox, p_acc


def algorithmic_flops(w, p_bbox, p_acc, filled_slots):
    """fp32 flops per pair (edge functions 15, barycentrics 3, three
    point-segment distances 33, clip, renormalisation and depth 11): with a
    blur radius every box pair needs the distances (51 per box pair, 11 per
    candidate); without one they are only needed for the output slots (18
    per box pair, 11 per candidate, 33 per filled slot). Backward: about 140
    per filled slot. Top-K compares and selects are not flops."""
    if w.blur > 0:
        fwd = 51 * p_bbox + 11 * p_acc
    else:
        fwd = 18 * p_bbox + 11 * p_acc + 33 * filled_slots
    return {"fwd": fwd, "bwd": 140 * filled_slots}


# ---------------------------------------------------------------------------
# traffic counters (rocprofv3 FETCH_SIZE / WRITE_SIZE summaries)
# ---------------------------------------------------------------------------

# Sources each timed kernel is built from: a traffic measurement is used only
# while these files are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "fine_raster": ("raster_fwd.hip", "dmr_internal.h"),
    "backward_slots": ("raster_bwd.hip", "dmr_internal.h", "lds_accum.h"),
}


def kernel_source_digest(kernel: str) -> str:
    import hashlib

    csrc = os.path.join(HERE, "differentiable_mesh_rasterization_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this
    kernel and workload (FETCH_SIZE + WRITE_SIZE, calibrated against a plain
    copy), or None when there is none or the kernel's sources changed since."""
    path = os.path.join(HERE, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("DATA "):
                fields = dict(kv.split("=", 1) for kv in line.split()[1:])
    if fields.get("source") != kernel_source_digest(kernel):
        return None
    return int(float(fields["fetch_bytes"]) + float(fields["write_bytes"]))


def copy_calibration(nbytes: int, reps: int) -> None:
    """Kernels of known traffic, for calibrating the HBM byte counters (run
    under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE): a plain device copy
    (reads and writes nbytes), a sum (reads nbytes, 16-byte loads) and a
    fill (writes nbytes). Two kernels that read the same bytes with
    different request patterns check that one scale fits both."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    for _ in range(reps):
        dst.copy_(src)
    for _ in range(reps):
        torch.sum(src, dim=0, out=acc)
    for _ in range(reps):
        dst.fill_(2.0)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "reps": reps}), flush=True)


# ---------------------------------------------------------------------------
# device inputs and timing
# ---------------------------------------------------------------------------

class DeviceCase:
    """One workload's inputs, outputs, upstream gradients and workspace in
    HBM. The upstream gradients are N(0, 1) over every slot for the
    gradients the workload drives, drawn on the device from a fixed seed
    (their values do not change the work; the parity checks draw their own
    on the host)."""

    def __init__(self, dmr, torch, w, dev):
        self.dmr, self.torch, self.w, self.dev = dmr, torch, w, dev
        t = lambda a: torch.from_numpy(a).to(dev)
        self.verts, self.faces, self.offsets = t(w.verts), t(w.faces), t(w.offsets)
        shape = (w.N, w.H, w.W, w.K)
        self.out = (torch.empty(shape, dtype=torch.int64, device=dev),
                    torch.empty(shape, dtype=torch.float32, device=dev),
                    torch.empty(shape + (3,), dtype=torch.float32, device=dev),
                    torch.empty(shape, dtype=torch.float32, device=dev))
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.grad_seed)
        self.g = {}
        for k in ("zbuf", "bary", "dists"):
            tail = (3,) if k == "bary" else ()
            self.g[k] = torch.randn(shape + tail, generator=gen, device=dev) if k in w.grads else None
        self.gv = torch.empty_like(self.verts)
        self.ws = dmr.Workspace(dev)
        self.ws.ensure(dmr.dmr_workspace_size_hint(w.N, w.F, w.H, w.W, w.K, w.blur))

    def fwd(self):
        w = self.w
        self.dmr.rasterize_meshes_fwd(self.verts, self.faces, self.offsets, w.H, w.W, w.K, w.blur, *self.out,
                                      self.ws.buf)

    def bwd(self, g=None):
        w = self.w
        g = self.g if g is None else g
        # the backward pass reuses the forward pass's face records and bin lists
        self.dmr.rasterize_meshes_bwd(self.verts, self.faces, self.offsets, w.H, w.W, w.K, w.blur, self.out[0],
                                      g["zbuf"], g["bary"], g["dists"], self.gv, self.ws.buf,
                                      reuse_forward_workspace=True)

    def step(self):
        self.fwd()
        self.bwd()

    def prepare(self, warmup: int):
        self.fwd()
        self.ws.grow()   # size the workspace so every bin list fits
        for _ in range(max(1, warmup)):
            self.step()
        self.torch.cuda.synchronize()


def timed(torch, fn, steps: int):
    """Mean ms per call of fn over `steps` calls: the larger of the HIP-event
    time on the current stream and the host wall time, both bracketed by a
    device synchronisation."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return max(e0.elapsed_time(e1) / steps, (t1 - t0) * 1e3 / steps)


def kernel_breakdown(dmr, torch, fn, steps: int):
    """Mean µs per launch of every kernel, from HIP events around each launch
    (a separate untimed run)."""
    dmr.set_kernel_timing(True)
    dmr.reset_kernel_timing()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    kt = dmr.kernel_timing()
    dmr.set_kernel_timing(False)
    return {k: round(ms / n * 1e3, 2) for k, (ms, n) in kt.items() if n}


def fractions(nbytes, flops, ms):
    s = ms * 1e-3
    return {"hbm_frac": round(nbytes / s / 1e9 / HBM_PEAK_GBS, 4),
            "valu_frac": round(flops / s / 1e12 / VALU_PEAK_TFLOPS, 5),
            "valu_frac_unpacked": round(flops / s / 1e12 / VALU_UNPACKED_TFLOPS, 5)}


def measure_config(dmr, torch, w, dev, steps: int, warmup: int):
    """Forward-only and forward+backward throughput of one workload, with the
    HBM and fp32-VALU fractions of its algorithmic work and its kernel
    times."""
    c = DeviceCase(dmr, torch, w, dev)
    c.prepare(warmup)
    n = steps if w.slots <= 100_000_000 else max(3, steps // 4)
    fwd_ms = timed(torch, c.fwd, n)
    step_ms = timed(torch, c.step, n)
    kernels = kernel_breakdown(dmr, torch, c.step, min(n, 5))
    filled = int((c.out[0] >= 0).sum().item())
    stats = dmr.dmr_workspace_stats(c.ws.buf)
    p_bbox, p_acc = pair_counts(w)
    nb = algorithmic_bytes(w, filled)
    fl = algorithmic_flops(w, p_bbox, p_acc, filled)
    f_fwd = fractions(nb["fwd_total"], fl["fwd"], fwd_ms)
    f_step = fractions(nb["fwd_total"] + nb["bwd_total"], fl["fwd"] + fl["bwd"], step_ms)
    floor_hbm = (nb["fwd_total"] + nb["bwd_total"]) / (HBM_PEAK_GBS * 1e9)
    floor_valu = (fl["fwd"] + fl["bwd"]) / (VALU_PEAK_TFLOPS * 1e12)
    res = {
        "N": w.N, "H": w.H, "W": w.W, "K": w.K, "blur_radius": w.blur, "faces": w.F, "verts": w.V,
        "slots": w.slots, "filled_slots": filled, "grads": list(w.grads),
        "fwd_ms": round(fwd_ms, 4), "fwd_bwd_ms": round(step_ms, 4), "bwd_ms": round(step_ms - fwd_ms, 4),
        "fwd_value": round(w.slots / (fwd_ms * 1e-3) / 1e6, 1),
        "fwd_bwd_value": round(w.slots / (step_ms * 1e-3) / 1e6, 1), "unit": "Mpix*K/s",
        "fwd": f_fwd, "fwd_bwd": f_step,
        "binding": "hbm" if floor_hbm >= floor_valu else "valu",
        "algorithmic_bytes": {"fwd": nb["fwd_total"], "bwd": nb["bwd_total"]},
        "algorithmic_flops": {"fwd": fl["fwd"], "bwd": fl["bwd"], "P_bbox": p_bbox, "P_acc_est": p_acc},
        "kernels_us": kernels,
        "workspace": {k: stats[k] for k in ("required_bytes", "bin_entries", "overflow_bins", "live_faces")},
    }
    return res, c


# ---------------------------------------------------------------------------
# the CPU oracle beside the GPU: baseline timing and parity on samples
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity_on_sample(dmr, torch, c, pix, ref_fwd, ref_p2f_for_grads=None):
    """GPU outputs against the oracle's on the sampled pixels `pix` (flat
    pixel ids): pix_to_face bit for bit except near-threshold pixels (the
    excuse rule), zbuf, bary and dists within 1e-5 on matching slots; then
    the backward pass with upstream gradients on the sampled pixels only,
    against the oracle's sum over them (relative L2)."""
    import numpy as np

    sys.path.insert(0, os.path.join(HERE, "tests"))
    import oracle
    from parity import compare_forward, oracle_excuse, rel_l2
    from workloads import masked_upstream_grads

    w = c.w
    idx = torch.from_numpy(pix).to(c.dev)
    got = tuple(t.reshape((-1, w.K) + tuple(t.shape[4:])).index_select(0, idx).cpu().numpy() for t in c.out)
    rep = compare_forward(ref_fwd, got, w.K,
                          excuse=oracle_excuse(oracle, w.verts, w.faces, w.offsets, w.H, w.W, w.blur, pixel_ids=pix))
    # backward: upstream gradients on the sampled pixels only
    sg = masked_upstream_grads(w, pix)
    shape = (w.N, w.H, w.W, w.K)
    dense = {}
    for key in ("zbuf", "bary", "dists"):
        if sg[key] is None:
            dense[key] = None
            continue
        tail = (3,) if key == "bary" else ()
        full = torch.zeros(shape + tail, dtype=torch.float32, device=c.dev)
        full.view((-1, w.K) + tail).index_copy_(0, idx, torch.from_numpy(sg[key]).to(c.dev))
        dense[key] = full
    c.bwd(dense)
    gv = c.gv.cpu().numpy()
    del dense
    ref_g = oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, ref_fwd[0],
                            sg["zbuf"], sg["bary"], sg["dists"], pixels=pix)
    return {"pixels": rep["pixels"], "excused": len(rep["excused"]), "unexcused": len(rep["unexcused"]),
            "excused_frac": len(rep["excused"]) / max(1, rep["pixels"]),
            "max_err_zbuf": rep["max_err_zbuf"], "max_err_bary": rep["max_err_bary"],
            "max_err_dists": rep["max_err_dists"], "padding_ok": rep["padding_ok"],
            "filled_slots": rep["filled_slots"], "grad_rel_l2": rel_l2(gv, ref_g),
            "ok": bool(not rep["unexcused"] and rep["values_ok"] and rep["padding_ok"]
                       and len(rep["excused"]) <= 1e-4 * rep["pixels"] and rel_l2(gv, ref_g) <= 1e-4)}


def cpu_baseline(dmr, torch, c, seconds: float):
    """The oracle, as it stands, on a bounded random sample of the workload's
    pixels (forward, then backward with the sample's upstream gradients);
    its outputs then serve the parity check of the same sample."""
    import numpy as np

    import oracle

    w = c.w
    rng = np.random.Generator(np.random.PCG64(99))
    gz = None if c.g["zbuf"] is None else c.g["zbuf"]
    chunks, t_fwd, t_bwd = [], 0.0, 0.0
    batch = 256
    while t_fwd + t_bwd < seconds:
        pix = np.unique(rng.integers(0, w.pixels, batch))
        t0 = time.perf_counter()
        ref = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, pixels=pix)
        t1 = time.perf_counter()
        sel = {}
        for k in ("zbuf", "bary", "dists"):
            t = c.g[k]
            sel[k] = None if t is None else t.reshape((w.pixels, w.K) + tuple(t.shape[4:])).index_select(
                0, torch.from_numpy(pix).to(c.dev)).cpu().numpy()
        t2 = time.perf_counter()
        oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, ref[0],
                        sel["zbuf"], sel["bary"], sel["dists"], pixels=pix)
        t3 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t3 - t2
        chunks.append((pix, ref))
        batch = min(batch * 2, 65536)
    # one sample of distinct pixels for the parity check
    allpix = np.concatenate([p for p, _ in chunks])
    order = np.argsort(allpix, kind="stable")
    keep = order[np.concatenate([[True], np.diff(allpix[order]) != 0])]
    refs = tuple(np.concatenate([r[i] for _, r in chunks])[keep] for i in range(4))
    slots = len(allpix) * w.K
    base = {
        "value": slots / (t_fwd + t_bwd) / 1e6,
        "unit": "Mpix*K/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{len(allpix)} uniformly drawn pixels of {w.name} ({slots} slots), "
                  f"fwd {t_fwd:.1f} s + bwd {t_bwd:.1f} s on the host CPU",
        "fwd_value": slots / t_fwd / 1e6,
    }
    return base, allpix[keep], refs


# per workload: pixels the oracle compares (None: every pixel)
PARITY_SAMPLE = {"sphere64": None, "spheres8_137": None, "soup1m_1024": 1500, "soups32_512": 12000}


def suite_parity(dmr, torch, c):
    """Parity of one suite workload on its sample (the headline workload is
    checked on the cpu_baseline sample instead)."""
    import numpy as np

    import oracle
    from workloads import sample_pixels

    w = c.w
    n = PARITY_SAMPLE[w.name]
    pix = np.arange(w.pixels, dtype=np.int64) if n is None else sample_pixels(w, n, seed=31)
    ref = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, pixels=pix)
    return parity_on_sample(dmr, torch, c, pix, ref)


# ---------------------------------------------------------------------------
# the rows beyond the path, measured after the timed step
# ---------------------------------------------------------------------------

def blend_measurement(dmr, torch, w, p2f, zbuf, dists, dev, steps):
    """The second stage (the K slots fused into RGBA) on the step's outputs,
    forward and backward, timed with HIP events outside the timed step, with
    its HBM roofline: 16 B per slot read (index, depth, distance), the face
    colours once and 16 B per pixel written (forward); the backward also
    reads 16 B and writes 8 B per slot."""
    from workloads import blend_upstream_grads, face_colors

    colors = torch.from_numpy(face_colors(w)).to(dev)
    grad = torch.from_numpy(blend_upstream_grads(w)).to(dev)
    prm = dmr.blend_params()
    rgba = torch.empty(p2f.shape[:-1] + (4,), dtype=torch.float32, device=dev)
    gz = torch.empty_like(zbuf)
    gd = torch.empty_like(dists)
    for _ in range(2):
        dmr.dmr_blend_fwd(p2f, zbuf, dists, colors, prm, rgba)
        dmr.dmr_blend_bwd(p2f, zbuf, dists, colors, prm, grad, gz, gd)
    torch.cuda.synchronize()
    dmr.set_kernel_timing_only(["blend_fwd", "blend_bwd"])
    dmr.reset_kernel_timing()
    for _ in range(steps):
        dmr.dmr_blend_fwd(p2f, zbuf, dists, colors, prm, rgba)
        dmr.dmr_blend_bwd(p2f, zbuf, dists, colors, prm, grad, gz, gd)
    torch.cuda.synchronize()
    kt = dmr.kernel_timing()
    dmr.set_kernel_timing(False)
    pixels = w.pixels
    fwd_bytes = 16 * w.slots + 12 * w.F + 16 * pixels
    bwd_bytes = 16 * w.slots + 12 * w.F + 16 * pixels + 8 * w.slots
    out = {}
    for name, nbytes in (("blend_fwd", fwd_bytes), ("blend_bwd", bwd_bytes)):
        ms, n = kt[name]
        us = ms / n * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"avg_us": round(us, 2), "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    out["value"] = round(w.slots / ((out["blend_fwd"]["avg_us"] + out["blend_bwd"]["avg_us"]) * 1e-6) / 1e6, 1)
    out["unit"] = "Mpix*K/s"
    return out


def projection_measurement(dmr, torch, w, dev, steps):
    """The upstream projection of the workload's meshes (world space to
    NDC through one camera per mesh), forward and backward with the camera
    gradient, timed with HIP events outside the timed step, with its HBM
    roofline: 12 B per vertex read and 12 B written (forward); 24 B read and
    12 B written (backward), plus the cameras."""
    from workloads import projection_inputs, projection_upstream_grads

    X, vo, M = projection_inputs(w)
    Xd = torch.from_numpy(X).to(dev)
    vod = torch.from_numpy(vo).to(dev)
    Md = torch.from_numpy(M).to(dev)
    gd = torch.from_numpy(projection_upstream_grads(w)).to(dev)
    out = torch.empty_like(Xd)
    gv = torch.empty_like(Xd)
    gc = torch.empty_like(Md)

    def run():
        dmr.dmr_project_fwd(Xd, vod, Md, out)
        dmr.dmr_project_bwd(Xd, vod, Md, gd, gv, gc)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    dmr.set_kernel_timing_only(["project_fwd", "project_bwd"])
    dmr.reset_kernel_timing()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    kt = dmr.kernel_timing()
    dmr.set_kernel_timing(False)
    cams = 64 * w.N + 8 * (w.N + 1)
    res = {}
    for name, nbytes in (("project_fwd", 24 * w.V + cams), ("project_bwd", 36 * w.V + 2 * cams)):
        ms, n = kt[name]
        us = ms / n * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"avg_us": round(us, 2), "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    res["vertices"] = w.V
    return res


def points_measurement(dmr, torch, dev, steps):
    """Point-cloud rasterization of the 16 clouds of the same spheres' vertices
    (225,312 points) at 256x256, K = 10, radius 0.01 NDC: forward + backward
    per step timed with events, and the fine pass's HBM roofline (16 B per
    slot written: index, depth, distance; 16 B per live point read)."""
    from workloads import make_point_workload, point_upstream_grads

    w = make_point_workload("points16_256")
    pts = torch.from_numpy(w.points).to(dev)
    off = torch.from_numpy(w.offsets).to(dev)
    g = {k: torch.from_numpy(v).to(dev) for k, v in point_upstream_grads(w).items()}
    shape = (w.N, w.H, w.W, w.K)
    idx = torch.empty(shape, dtype=torch.int64, device=dev)
    zb = torch.empty(shape, dtype=torch.float32, device=dev)
    ds = torch.empty(shape, dtype=torch.float32, device=dev)
    gp = torch.empty_like(pts)
    ws = torch.empty(dmr.dmr_points_workspace_size_hint(w.N, w.P, w.H, w.W, w.K, w.radius), dtype=torch.uint8,
                     device=dev)

    def step():
        dmr.rasterize_points_fwd(pts, off, w.H, w.W, w.K, w.radius, idx, zb, ds, ws)
        dmr.rasterize_points_bwd(pts, off, w.H, w.W, w.K, idx, g["zbuf"], g["dists"], gp)

    for _ in range(2):
        step()
    ms = timed(torch, step, steps)
    kt = kernel_breakdown(dmr, torch, step, min(steps, 10))
    live = dmr.dmr_workspace_stats(ws)["live_faces"]
    kernels = {k: v for k, v in kt.items() if k in
               ("zero_fwd", "point_setup", "bin_scan", "bin_fill", "bin_sort", "point_raster", "point_bwd")}
    fine_bytes = 16 * w.slots + 16 * live
    fine_us = kernels.get("point_raster")
    return {"workload": "points16_256", "points": w.P, "slots": w.slots,
            "filled_slots": int((idx >= 0).sum().item()), "ms_per_step": round(ms, 4),
            "value": round(w.slots / (ms * 1e-3) / 1e6, 1), "unit": "Mpix*K/s", "kernels_us": kernels,
            "point_raster_hbm_frac": None if not fine_us else round(fine_bytes / (fine_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                                                     4)}


def settings_measurement(dmr, torch, c, steps):
    """The same step under each rasterizer setting (perspective-correct
    barycentrics, back-face culling, unclipped barycentrics, all three),
    timed with events outside the timed step: ms per step and Mpix*K/s."""
    w = c.w
    variants = {"perspective_correct": dmr.DMR_RASTER_PERSPECTIVE_CORRECT,
                "cull_backfaces": dmr.DMR_RASTER_CULL_BACKFACES,
                "unclipped_bary": dmr.DMR_RASTER_UNCLIPPED_BARY,
                "all_three": (dmr.DMR_RASTER_PERSPECTIVE_CORRECT | dmr.DMR_RASTER_CULL_BACKFACES
                              | dmr.DMR_RASTER_UNCLIPPED_BARY)}
    out = {}
    for name, flags in variants.items():
        def step():
            dmr.rasterize_meshes_fwd_ex(c.verts, c.faces, c.offsets, w.H, w.W, w.K, w.blur, *c.out, c.ws.buf, flags)
            dmr.rasterize_meshes_bwd(c.verts, c.faces, c.offsets, w.H, w.W, w.K, w.blur, c.out[0], c.g["zbuf"],
                                     c.g["bary"], c.g["dists"], c.gv, c.ws.buf, reuse_forward_workspace=True,
                                     settings=flags)

        for _ in range(2):
            step()
        ms = timed(torch, step, steps)
        out[name] = {"ms_per_step": round(ms, 4), "value": round(w.slots / (ms * 1e-3) / 1e6, 1),
                     "filled_slots": int((c.out[0] >= 0).sum().item())}
    out["unit"] = "Mpix*K/s"
    return out


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hetero16_256")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (baseline and parity)")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-suite", action="store_true", help="skip the per-workload suite")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements after the timed step (second stage, projection, point clouds, "
                         "rasterizer settings)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(each image is independent; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    import torch

    import differentiable_mesh_rasterization_amd as dmr
    from workloads import make_workload

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = make_workload(args.workload)
    c = DeviceCase(dmr, torch, w, dev)
    c.prepare(args.warmup)
    stats = dmr.dmr_workspace_stats(c.ws.buf)
    filled = int((c.out[0] >= 0).sum().item())

    # The per-kernel breakdown (a separate, untimed run with events around
    # every launch) names the dominant kernel of the two that can dominate
    # (the fine pass and the backward pass). In the timed region HIP events
    # bracket that kernel only, on the stream it runs on: each event record
    # costs the step a few microseconds.
    dominant_candidates = ("fine_raster", "backward_slots")
    kernels = {}
    dominant = None
    if not args.no_kernel_timing:
        kernels = kernel_breakdown(dmr, torch, c.step, min(args.steps, 10))
        dominant = max(dominant_candidates, key=lambda k: kernels.get(k, 0.0))
        dmr.set_kernel_timing_only((dominant,))
        dmr.reset_kernel_timing()
    ms_per_step = timed(torch, c.step, args.steps)
    kt = dmr.kernel_timing() if not args.no_kernel_timing else {}
    dmr.set_kernel_timing(False)
    value = w.slots / (ms_per_step * 1e-3) / 1e6

    nb = algorithmic_bytes(w, filled)
    p_bbox, p_acc = pair_counts(w)
    fl = algorithmic_flops(w, p_bbox, p_acc, filled)
    roofline = None
    if kt and dominant in kt and kt[dominant][1] > 0:
        ms, n = kt[dominant]
        avg_s = ms / n * 1e-3
        achieved = nb[dominant] / avg_s / 1e9
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(dominant, w.name),
                    "algorithmic_bytes_per_launch": nb[dominant], "avg_launch_us": round(avg_s * 1e6, 2)}
    step_s = ms_per_step * 1e-3
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "Mpix*K/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "H": w.H, "W": w.W, "K": w.K, "blur_radius": w.blur,
                   "faces": w.F, "verts": w.V, "slots": w.slots, "filled_slots": filled,
                   "grads": list(w.grads), "parallelism": "single GPU"},
        "roofline": roofline,
        "valu": {"bound": "valu", "achieved": round((fl["fwd"] + fl["bwd"]) / step_s / 1e12, 3),
                 "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round((fl["fwd"] + fl["bwd"]) / step_s / 1e12 / VALU_PEAK_TFLOPS, 5),
                 "peak_unpacked": VALU_UNPACKED_TFLOPS,
                 "frac_unpacked": round((fl["fwd"] + fl["bwd"]) / step_s / 1e12 / VALU_UNPACKED_TFLOPS, 5),
                 "flops_per_step": fl["fwd"] + fl["bwd"], "P_bbox": p_bbox, "P_acc_est": p_acc},
        "kernels": kernels,
        "fwd_bwd_hbm_frac": round((nb["fwd_total"] + nb["bwd_total"]) / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "workspace": {k: stats[k] for k in ("required_bytes", "bin_entries", "overflow_bins", "live_faces")},
    }
    if not args.no_extras:
        line["blend"] = blend_measurement(dmr, torch, w, c.out[0], c.out[1], c.out[3], dev, args.steps)
        line["projection"] = projection_measurement(dmr, torch, w, dev, args.steps)
        line["points"] = points_measurement(dmr, torch, dev, args.steps)
        line["settings"] = settings_measurement(dmr, torch, c, args.steps)
    parity = {}
    if not args.no_cpu_baseline:
        c.step()   # the default outputs again (the settings runs overwrote them)
        torch.cuda.synchronize()
        base, pix, refs = cpu_baseline(dmr, torch, c, args.cpu_seconds)
        line["cpu_baseline"] = base
        parity[w.name] = parity_on_sample(dmr, torch, c, pix, refs)
    del c
    torch.cuda.empty_cache()
    if not args.no_suite:
        suite = {}
        for name in SUITE:
            ws = make_workload(name)
            res, cc = measure_config(dmr, torch, ws, dev, args.steps, args.warmup)
            if not args.no_cpu_baseline and name in PARITY_SAMPLE:
                parity[name] = suite_parity(dmr, torch, cc)
            suite[name] = res
            del cc
            torch.cuda.empty_cache()
        line["configs"] = suite
    if parity:
        line["parity"] = parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark: forward+backward K-nearest-face mesh rasterization on one MI355X.

One step = rasterize_meshes_fwd + rasterize_meshes_bwd (every stage of the
path: face setup, bin count, scan, bin fill, fine raster, gradient zeroing,
backward) over one batch of seeded synthetic meshes already resident in HBM.
The default workload is a heterogeneous batch of 16 icospheres (levels 3-6,
1280-81920 triangles each) at 256x256, K = 10, blur_radius = 1e-4.

Prints one JSON line: throughput in Mpixel*K slots per second, the roofline
of the dominant kernel (timed with HIP events on the stream it runs on,
inside the timed region; the other kernels' times come from a separate
untimed run), and the CPU oracle timed on a bounded pixel sample of the same
workload on this host.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload hetero16_256]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s

METRIC = "forward+backward Mpixels*K/s at 1 MI355X; % of fp32-VALU/HBM roofline"


def algorithmic_bytes(w, filled_slots, live_faces, grads):
    """Bytes each kernel must move at minimum (per launch)."""
    slots = w.slots
    fine = 28 * slots + 36 * live_faces  # outputs + face geometry read once
    g = (4 if "zbuf" in grads else 0) + (12 if "bary" in grads else 0) + (4 if "dists" in grads else 0)
    bwd = 8 * slots + g * filled_slots + 24 * w.F + 12 * w.V + 12 * w.V
    fwd_total = 28 * slots + 24 * w.F + 12 * w.V
    return {"fine_raster": fine, "backward_slots": bwd, "fwd_total": fwd_total, "bwd_total": bwd}


# Sources each timed kernel is built from: a traffic measurement is used only
# while these files are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "fine_raster": ("raster_fwd.hip", "dmr_internal.h"),
    "backward_slots": ("raster_bwd.hip", "dmr_internal.h", "lds_accum.h"),
}


def kernel_source_digest(kernel: str) -> str:
    import hashlib

    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "differentiable_mesh_rasterization_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this
    kernel and workload (FETCH_SIZE + WRITE_SIZE, calibrated against a plain
    copy), or None when there is none or the kernel's sources changed since."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{kernel}_{workload}_traffic.md")
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
    """A plain device copy of a known size, for calibrating the HBM byte
    counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "reps": reps}), flush=True)


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
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    dmr.set_kernel_timing(True)
    dmr.reset_kernel_timing()
    for _ in range(min(steps, 10)):
        step()
    torch.cuda.synchronize()
    kt = dmr.kernel_timing()
    dmr.set_kernel_timing(False)
    live = dmr.dmr_workspace_stats(ws)["live_faces"]
    kernels = {k: round(v[0] / v[1] * 1e3, 2) for k, v in kt.items() if v[1] and k in
               ("zero_fwd", "point_setup", "bin_scan", "bin_fill", "bin_sort", "point_raster", "point_bwd")}
    fine_bytes = 16 * w.slots + 16 * live
    fine_us = kernels.get("point_raster")
    return {"workload": "points16_256", "points": w.P, "slots": w.slots,
            "filled_slots": int((idx >= 0).sum().item()), "ms_per_step": round(ms, 4),
            "value": round(w.slots / (ms * 1e-3) / 1e6, 1), "unit": "Mpix*K/s", "kernels_us": kernels,
            "point_raster_hbm_frac": None if not fine_us else round(fine_bytes / (fine_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                                                     4)}


def settings_measurement(dmr, torch, w, verts, faces, offsets, g, outs, gv, ws, dev, steps):
    """The same step under each rasterizer setting (perspective-correct
    barycentrics, back-face culling, unclipped barycentrics, all three),
    timed with events outside the timed step: ms per step and Mpix*K/s."""
    variants = {"perspective_correct": dmr.DMR_RASTER_PERSPECTIVE_CORRECT,
                "cull_backfaces": dmr.DMR_RASTER_CULL_BACKFACES,
                "unclipped_bary": dmr.DMR_RASTER_UNCLIPPED_BARY,
                "all_three": (dmr.DMR_RASTER_PERSPECTIVE_CORRECT | dmr.DMR_RASTER_CULL_BACKFACES
                              | dmr.DMR_RASTER_UNCLIPPED_BARY)}
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, flags in variants.items():
        def step():
            dmr.rasterize_meshes_fwd_ex(verts, faces, offsets, w.H, w.W, w.K, w.blur, *outs, ws.buf, flags)
            dmr.rasterize_meshes_bwd(verts, faces, offsets, w.H, w.W, w.K, w.blur, outs[0], g["zbuf"], g["bary"],
                                     g["dists"], gv, ws.buf, reuse_forward_workspace=True, settings=flags)

        for _ in range(2):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[name] = {"ms_per_step": round(ms, 4), "value": round(w.slots / (ms * 1e-3) / 1e6, 1),
                     "filled_slots": int((outs[0] >= 0).sum().item())}
    out["unit"] = "Mpix*K/s"
    return out


def cpu_baseline(w, grads_np, seconds: float):
    """The oracle, as it stands, on a bounded sample of the workload's pixels."""
    import numpy as np

    import oracle
    from workloads import sample_pixels

    rng = np.random.Generator(np.random.PCG64(99))
    done_pix = 0
    t_fwd = t_bwd = 0.0
    batch = 256
    while t_fwd + t_bwd < seconds:
        pix = np.unique(rng.integers(0, w.pixels, batch))
        t0 = time.perf_counter()
        p2f = oracle.rasterize(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, pixels=pix)[0]
        t1 = time.perf_counter()
        sel = {k: (None if v is None else v.reshape((w.pixels, w.K) + v.shape[4:])[pix]) for k, v in grads_np.items()}
        oracle.backward(w.verts, w.faces, w.offsets, w.H, w.W, w.K, w.blur, p2f,
                        sel["zbuf"], sel["bary"], sel["dists"], pixels=pix)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t2 - t1
        done_pix += len(pix)
        batch = min(batch * 2, 65536)
    slots = done_pix * w.K
    return {
        "value": slots / (t_fwd + t_bwd) / 1e6,
        "unit": "Mpix*K/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{done_pix} uniformly drawn pixels of the same workload ({slots} slots), "
                  f"fwd {t_fwd:.1f} s + bwd {t_bwd:.1f} s on the host CPU",
        "fwd_value": slots / t_fwd / 1e6,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hetero16_256")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
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

    import numpy as np
    import torch

    import differentiable_mesh_rasterization_amd as dmr
    from workloads import make_workload, upstream_grads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = make_workload(args.workload)
    gnp = upstream_grads(w)
    stream = torch.cuda.current_stream(dev)

    verts = torch.from_numpy(w.verts).to(dev)
    faces = torch.from_numpy(w.faces).to(dev)
    offsets = torch.from_numpy(w.offsets).to(dev)
    shape = (w.N, w.H, w.W, w.K)
    p2f = torch.empty(shape, dtype=torch.int64, device=dev)
    zbuf = torch.empty(shape, dtype=torch.float32, device=dev)
    bary = torch.empty(shape + (3,), dtype=torch.float32, device=dev)
    dists = torch.empty(shape, dtype=torch.float32, device=dev)
    gv = torch.empty_like(verts)
    g = {k: (None if v is None else torch.from_numpy(v).to(dev)) for k, v in gnp.items()}
    ws = dmr.Workspace(dev)
    ws.ensure(dmr.dmr_workspace_size_hint(w.N, w.F, w.H, w.W, w.K, w.blur))

    def step():
        dmr.rasterize_meshes_fwd(verts, faces, offsets, w.H, w.W, w.K, w.blur, p2f, zbuf, bary, dists, ws.buf)
        # the backward pass reuses the forward pass's face records and bin lists
        dmr.rasterize_meshes_bwd(verts, faces, offsets, w.H, w.W, w.K, w.blur, p2f, g["zbuf"], g["bary"],
                                 g["dists"], gv, ws.buf, reuse_forward_workspace=True)

    step()
    stats = ws.grow()  # size the workspace so every bin list fits
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stats = dmr.dmr_workspace_stats(ws.buf)
    filled = int((p2f >= 0).sum().item())

    # Timed region: HIP events bracket the two kernels that can dominate
    # (the fine pass and the backward pass) on the stream they run on.
    dominant_candidates = ("fine_raster", "backward_slots")
    if not args.no_kernel_timing:
        dmr.set_kernel_timing_only(dominant_candidates)
        dmr.reset_kernel_timing()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = dmr.kernel_timing() if not args.no_kernel_timing else {}
    dmr.set_kernel_timing(False)
    ms_events = ev0.elapsed_time(ev1) / args.steps
    ms_wall = (t1 - t0) * 1e3 / args.steps
    ms_per_step = max(ms_events, ms_wall)
    value = w.slots / (ms_per_step * 1e-3) / 1e6

    # Per-kernel breakdown, after the timed region (every kernel bracketed).
    breakdown = {}
    if not args.no_kernel_timing:
        dmr.set_kernel_timing(True)
        dmr.reset_kernel_timing()
        for _ in range(min(args.steps, 10)):
            step()
        torch.cuda.synchronize()
        breakdown = dmr.kernel_timing()
        dmr.set_kernel_timing(False)

    alg = algorithmic_bytes(w, filled, stats["live_faces"], w.grads)
    kernels = {name: {"avg_us": round(ms / n * 1e3, 2) if n else None, "launches": n}
               for name, (ms, n) in breakdown.items()}
    roofline = None
    if kt:
        dominant = max(dominant_candidates, key=lambda k: kt[k][0])
        ms, n = kt[dominant]
        avg_s = ms / n * 1e-3
        achieved = alg[dominant] / avg_s / 1e9
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(dominant, w.name),
                    "algorithmic_bytes_per_launch": alg[dominant], "avg_launch_us": round(avg_s * 1e6, 2)}
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
        "kernels": kernels,
        "fwd_bwd_hbm_frac": round((alg["fwd_total"] + alg["bwd_total"]) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "workspace": {k: stats[k] for k in ("required_bytes", "bin_entries", "overflow_bins", "live_faces")},
    }
    if not args.no_extras:
        line["blend"] = blend_measurement(dmr, torch, w, p2f, zbuf, dists, dev, args.steps)
        line["projection"] = projection_measurement(dmr, torch, w, dev, args.steps)
        line["points"] = points_measurement(dmr, torch, dev, args.steps)
        line["settings"] = settings_measurement(dmr, torch, w, verts, faces, offsets, g, (p2f, zbuf, bary, dists),
                                                gv, ws, dev, args.steps)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, gnp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

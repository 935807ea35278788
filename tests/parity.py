"""Forward/backward comparison with the near-threshold excuse rule.

pix_to_face must match exactly. A pixel whose face list differs is excused
only when every face involved sits at a near-threshold point: its inclusion
flips when blur_radius moves by +-1e-6 (its squared distance is within 1e-6
of blur_radius), its depth is within 1e-6 of another candidate's depth (an
order swap, including across the K-th slot), or its depth is within 1e-6 of
zero (the z <= 0 skip). Values (zbuf, bary, dists) are compared on slots whose
face matches; padding must be exactly -1.
"""

from __future__ import annotations

import numpy as np

DELTA = 1e-6


def _rows(a, K, trailing=0):
    a = np.asarray(a)
    return a.reshape((-1, K) + a.shape[a.ndim - trailing:] if trailing else (-1, K))


def compare_forward(ref, got, K: int, atol: float = 1e-5, excuse=None):
    rp, rz, rb, rd = ref
    gp, gz, gb, gd = got
    rp, gp = _rows(rp, K), _rows(gp, K)
    rz, gz = _rows(rz, K), _rows(gz, K)
    rd, gd = _rows(rd, K), _rows(gd, K)
    rb, gb = _rows(rb, K, 1), _rows(gb, K, 1)
    assert rp.shape == gp.shape, (rp.shape, gp.shape)
    mism = np.nonzero((rp != gp).any(axis=1))[0]
    excused, unexcused = [], []
    for r in mism:
        ok = excuse is not None and excuse(int(r), rp[r], gp[r], rz[r], gz[r])
        (excused if ok else unexcused).append(int(r))
    same = (rp == gp) & (rp >= 0)
    pad = (rp == gp) & (rp < 0)

    def maxerr(a, b, m):
        # a NaN on both sides is a match (faces whose arithmetic meets NaN
        # give it on both sides); a NaN on one side is an infinite error
        if not m.any():
            return 0.0
        x, y = a[m].astype(np.float64), b[m].astype(np.float64)
        d = np.abs(x - y)
        d[np.isnan(x) & np.isnan(y)] = 0.0
        d[np.isnan(d)] = np.inf
        return float(np.max(d))

    rep = {
        "pixels": int(rp.shape[0]),
        "excused": excused,
        "unexcused": unexcused,
        "max_err_zbuf": maxerr(rz, gz, same),
        "max_err_bary": maxerr(rb, gb, same[..., None].repeat(3, -1)),
        "max_err_dists": maxerr(rd, gd, same),
        "padding_ok": bool(np.all(gz[pad] == -1) and np.all(gb[pad] == -1) and np.all(gd[pad] == -1)),
        "filled_slots": int(same.sum()),
    }
    rep["values_ok"] = (rep["max_err_zbuf"] <= atol and rep["max_err_bary"] <= atol
                        and rep["max_err_dists"] <= atol)
    return rep


def assert_forward_parity(rep, max_excused_frac: float = 1e-4):
    assert not rep["unexcused"], f"unexcused pix_to_face mismatches at rows {rep['unexcused'][:20]}"
    assert len(rep["excused"]) <= max_excused_frac * rep["pixels"], \
        f"{len(rep['excused'])} excused pixels of {rep['pixels']}"
    assert rep["padding_ok"], "padding slots are not exactly -1"
    assert rep["values_ok"], {k: rep[k] for k in ("max_err_zbuf", "max_err_bary", "max_err_dists")}


def _diff_faces(ref_faces, got_faces):
    """Faces that are missing on one side, or present on both in other slots."""
    out = set(int(f) for f in set(ref_faces.tolist()) ^ set(got_faces.tolist()) if f >= 0)
    for k, (a, b) in enumerate(zip(ref_faces, got_faces)):
        if a != b:
            if a >= 0:
                out.add(int(a))
            if b >= 0:
                out.add(int(b))
    return out


def oracle_excuse(oracle, w_verts, w_faces, w_offsets, H, W, blur, pixel_ids=None, delta=DELTA, settings=0):
    """Excuse function backed by the binary32 oracle (with the given
    rasterizer settings): pixel rows index pixel_ids (or all pixels in order
    when pixel_ids is None)."""
    offsets = np.asarray(w_offsets)

    def fn(row, ref_faces, got_faces, ref_z, got_z):
        pid = int(row if pixel_ids is None else pixel_ids[row])
        n = pid // (H * W)
        Kall = max(1, int(offsets[n + 1] - offsets[n]))
        runs = {}
        for tag, b in (("mid", blur), ("lo", max(0.0, blur - delta)), ("hi", blur + delta)):
            p, z, _, _ = oracle.rasterize(w_verts, w_faces, offsets, H, W, Kall, b,
                                          pixels=np.asarray([pid]), settings=settings)
            m = p[0] >= 0
            runs[tag] = dict(zip(p[0][m].tolist(), z[0][m].tolist()))
        near_blur = set(runs["hi"]) - set(runs["lo"])
        zmap = dict(runs["mid"])
        for f, z in zip(got_faces.tolist(), got_z.tolist()):
            if f >= 0 and f not in zmap:
                zmap[f] = z
        for f in _diff_faces(ref_faces, got_faces):
            if f in near_blur:
                continue
            zf = zmap.get(f)
            if zf is None:
                return False
            if abs(zf) <= delta:
                continue
            if any(abs(zf - zg) <= delta for g, zg in zmap.items() if g != f):
                continue
            return False
        return True

    return fn


def exact_excuse(details, N, H, W, blur, delta=DELTA):
    """Excuse function backed by exact per-face details (tests/exact_raster.py)."""
    from fractions import Fraction as Fr

    blur = Fr(float(np.float32(blur)))
    d = Fr(delta)

    def fn(row, ref_faces, got_faces, ref_z, got_z):
        n, rem = divmod(row, H * W)
        i, j = divmod(rem, W)
        per_face = details[(n, i, j)]
        cand_z = {f: r["z"] for f, r in per_face.items() if r["candidate"]}
        for f in _diff_faces(ref_faces, got_faces):
            r = per_face.get(f)
            if r is None:
                return False
            if abs(r["d2"] - blur) <= d:
                continue
            if abs(r["z"]) <= d:
                continue
            if any(abs(r["z"] - zg) <= d for g, zg in cand_z.items() if g != f):
                continue
            return False
        return True

    return fn


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def region_faces(verts, faces, offsets, n, H, W, blur, i0, i1, j0, j1, margin=1e-3):
    """Global ids (ascending) of mesh n's faces whose box, grown by
    sqrt(blur_radius) + margin, reaches the pixel centres of rows [i0, i1)
    and columns [j0, j1). A face outside that box is neither strictly inside
    at those pixels nor within sqrt(blur_radius) of them, so it cannot be a
    candidate there; the margin, far above binary32 rounding, keeps the
    selection conservative."""
    f0, f1 = int(offsets[n]), int(offsets[n + 1])
    tri = np.asarray(verts, np.float64)[np.asarray(faces[f0:f1], np.int64)]
    r = np.sqrt(blur) + margin
    xl = (2.0 * j0 + 1.0) / W - 1.0
    xh = (2.0 * (j1 - 1) + 1.0) / W - 1.0
    yl = (2.0 * i0 + 1.0) / H - 1.0
    yh = (2.0 * (i1 - 1) + 1.0) / H - 1.0
    keep = ((tri[..., 0].min(1) - r <= xh) & (tri[..., 0].max(1) + r >= xl)
            & (tri[..., 1].min(1) - r <= yh) & (tri[..., 1].max(1) + r >= yl))
    return f0 + np.nonzero(keep)[0]


def oracle_region(oracle, verts, faces, offsets, n, H, W, K, blur, i0, i1, j0, j1, grads=None, settings=0):
    """The oracle on the pixels of rows [i0, i1) x columns [j0, j1) of image
    n, run on the faces that can reach them (region_faces): the kept faces
    form one mesh in their global order, so depth ties break as in the
    whole batch, and their local indices map back to global ids.

    Returns (flat global pixel ids in row-major order, (pix_to_face, zbuf,
    bary, dists) for those pixels, and, with grads = (gz, gb, gd) shaped
    like the outputs (or None each), the oracle's grad_verts [V, 3] over
    them). `settings` (the oracle's setting bits) applies to both passes:
    culling and perspective correction only remove or reweight candidates
    that the region's box test already bounds, so the reduction holds under
    every setting."""
    kept = region_faces(verts, faces, offsets, n, H, W, blur, i0, i1, j0, j1)
    sub = np.ascontiguousarray(np.asarray(faces, np.int64)[kept])
    ii, jj = np.meshgrid(np.arange(i0, i1), np.arange(j0, j1), indexing="ij")
    local = (ii * W + jj).reshape(-1).astype(np.int64)
    sub_off = np.array([0, len(kept)], np.int64)
    p2f, zb, ba, ds = oracle.rasterize(verts, sub, sub_off, H, W, K, blur, pixels=local, settings=settings)
    glob = np.append(kept, -1)[np.where(p2f >= 0, p2f, len(kept))]
    gv = None
    if grads is not None:
        gz, gb, gd = grads
        gv = oracle.backward(verts, sub, sub_off, H, W, K, blur, p2f, gz, gb, gd, pixels=local, settings=settings)
    return n * H * W + local, (glob, zb, ba, ds), gv


def point_oracle_band(rasterize_points, w, n, r0, r1, pts_np):
    """The oracle on rows [r0, r1) of image n, run on only the points of that
    image whose y lies within the radius (with margin) of the band's pixel
    centres, in their original order, so that ties by index order the same;
    the indices are mapped back to global ones. A point farther than the
    radius from every centre of the band is never a candidate there, so
    this equals the whole-image oracle on the band."""
    lo, hi = int(w.offsets[n]), int(w.offsets[n + 1])
    q = pts_np[lo:hi]
    yc = (np.arange(r0, r1, dtype=np.float64) * 2 + 1) / w.H - 1
    pad = 2.0 * w.radius + 1e-6
    keep = np.nonzero((q[:, 1] >= yc.min() - pad) & (q[:, 1] <= yc.max() + pad))[0]
    pix = (np.arange(r0, r1)[:, None] * w.W + np.arange(w.W)[None, :]).reshape(-1)
    idx, zb, ds = rasterize_points(q[keep], [0, len(keep)], w.H, w.W, w.K, w.radius, pixels=pix)
    gidx = np.full_like(idx, -1)
    if len(keep):
        gidx = np.where(idx >= 0, lo + keep[np.maximum(idx, 0)], -1)
    return gidx, zb, ds

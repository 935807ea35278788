"""Seeded synthetic mesh batches in screen space (x, y in NDC, z = view depth).

Every workload is drawn with numpy's PCG64 generator from a fixed seed, built in
float64 and rounded once to float32, so that the oracle and the GPU path read
the very same bits. Faces index the packed vertex array globally; mesh n owns
the faces [offsets[n], offsets[n+1]).

The pages describe heterogeneous batches of meshes with different vertex and
face counts (Accelerating 3D Deep Learning with PyTorch3D, gptget.net summary,
"Methodology"; rocketrecap video summary, "1:00 Heterogeneous Batching") and
name the icosphere primitive as a starting shape ("2:02 Data Structures and
I/O"). The ShapeNet experiments use 137x137 renders ("Experiments"); the
sphere-batch workload below borrows that image size.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

GRAD_NAMES = ("zbuf", "bary", "dists")


@dataclasses.dataclass
class Workload:
    name: str
    verts: np.ndarray  # [V, 3] float32
    faces: np.ndarray  # [F, 3] int64 (global vertex indices)
    offsets: np.ndarray  # [N + 1] int64
    H: int
    W: int
    K: int
    blur: float  # a float32 value, squared NDC units
    grads: tuple  # which upstream gradients the workload drives
    seed: int
    grad_seed: int

    @property
    def N(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def F(self) -> int:
        return int(self.faces.shape[0])

    @property
    def V(self) -> int:
        return int(self.verts.shape[0])

    @property
    def slots(self) -> int:
        return self.N * self.H * self.W * self.K

    @property
    def pixels(self) -> int:
        return self.N * self.H * self.W


# ----------------------------------------------------------------------------
# geometry helpers (float64)
# ----------------------------------------------------------------------------

def icosphere(level: int):
    """Unit icosphere: an icosahedron refined `level` times by 4-way midpoint
    subdivision, new vertices pushed to the unit sphere.

    Returns (verts [10*4^L+2, 3] float64, faces [20*4^L, 3] int64)."""
    phi = (1.0 + math.sqrt(5.0)) / 2.0
    v = [(-1, phi, 0), (1, phi, 0), (-1, -phi, 0), (1, -phi, 0),
         (0, -1, phi), (0, 1, phi), (0, -1, -phi), (0, 1, -phi),
         (phi, 0, -1), (phi, 0, 1), (-phi, 0, -1), (-phi, 0, 1)]
    verts = [np.array(p, dtype=np.float64) / math.sqrt(1.0 + phi * phi) for p in v]
    faces = [(0, 11, 5), (0, 5, 1), (0, 1, 7), (0, 7, 10), (0, 10, 11),
             (1, 5, 9), (5, 11, 4), (11, 10, 2), (10, 7, 6), (7, 1, 8),
             (3, 9, 4), (3, 4, 2), (3, 2, 6), (3, 6, 8), (3, 8, 9),
             (4, 9, 5), (2, 4, 11), (6, 2, 10), (8, 6, 7), (9, 8, 1)]
    for _ in range(level):
        cache = {}

        def mid(a, b):
            key = (a, b) if a < b else (b, a)
            if key not in cache:
                m = verts[a] + verts[b]
                verts.append(m / np.linalg.norm(m))
                cache[key] = len(verts) - 1
            return cache[key]

        nf = []
        for (a, b, c) in faces:
            ab, bc, ca = mid(a, b), mid(b, c), mid(c, a)
            nf += [(a, ab, ca), (b, bc, ab), (c, ca, bc), (ab, bc, ca)]
        faces = nf
    return np.stack(verts), np.asarray(faces, dtype=np.int64)


def _rotation(rng: np.random.Generator) -> np.ndarray:
    """Uniform random rotation from a normalised 4-vector (unit quaternion)."""
    q = rng.normal(size=4)
    w, x, y, z = q / np.linalg.norm(q)
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
        [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
        [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)],
    ])


def _fit(v: np.ndarray, xy_bound: float, z_lo: float, z_hi: float) -> np.ndarray:
    """Centre xy on the bounding-box midpoint, scale xy uniformly so that
    max(|x|, |y|) == xy_bound, and map z affinely from [min, max] to [z_lo, z_hi]."""
    v = v.copy()
    lo, hi = v.min(axis=0), v.max(axis=0)
    v[:, 0] -= 0.5 * (lo[0] + hi[0])
    v[:, 1] -= 0.5 * (lo[1] + hi[1])
    v[:, :2] *= xy_bound / np.abs(v[:, :2]).max()
    v[:, 2] = z_lo + (v[:, 2] - lo[2]) / (hi[2] - lo[2]) * (z_hi - z_lo)
    return v


def _pack(meshes):
    """meshes: list of (verts float64 [Vn,3], faces int64 [Fn,3] local) -> packed arrays."""
    vs, fs, offs = [], [], [0]
    vbase = 0
    for v, f in meshes:
        vs.append(v)
        fs.append(f + vbase)
        vbase += v.shape[0]
        offs.append(offs[-1] + f.shape[0])
    verts = np.concatenate(vs).astype(np.float32) if vs else np.zeros((0, 3), np.float32)
    faces = np.concatenate(fs).astype(np.int64) if fs else np.zeros((0, 3), np.int64)
    return verts, faces, np.asarray(offs, dtype=np.int64)


def _soup(rng, F, xy_lo, xy_hi, z_lo, z_hi, sigma, neg_frac=0.0, neg_z=(-0.5, -0.05)):
    """Triangle soup: F independent triangles, each vertex = centroid + N(0, sigma^2) per axis."""
    c = np.empty((F, 3))
    c[:, 0] = rng.uniform(xy_lo, xy_hi, F)
    c[:, 1] = rng.uniform(xy_lo, xy_hi, F)
    c[:, 2] = rng.uniform(z_lo, z_hi, F)
    if neg_frac > 0.0:
        neg = rng.random(F) < neg_frac
        c[neg, 2] = rng.uniform(neg_z[0], neg_z[1], int(neg.sum()))
    v = c[:, None, :] + rng.normal(0.0, sigma, (F, 3, 3))
    return v.reshape(-1, 3), np.arange(3 * F, dtype=np.int64).reshape(F, 3)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def _sphere64(rng):
    v, f = icosphere(2)
    v = v + rng.normal(0.0, 0.05, v.shape)
    v = v @ _rotation(rng).T
    return [(_fit(v, 0.8, 1.5, 2.5), f)], 64, 64, 1, 0.0, ("zbuf",)


def _spheres8(rng):
    base, f = icosphere(4)
    meshes = []
    for _ in range(8):
        v = base + rng.normal(0.0, 0.03, base.shape)
        v = v @ _rotation(rng).T
        meshes.append((_fit(v, 0.9, 1.0, 3.0), f))
    return meshes, 137, 137, 8, 1e-4, ("bary", "dists")


def _hetero16(rng):
    spheres = {L: icosphere(L) for L in (3, 4, 5, 6)}
    meshes = []
    for _ in range(16):
        L = int(rng.integers(3, 7))
        base, f = spheres[L]
        v = base * (1.0 + rng.normal(0.0, 0.05, (base.shape[0], 1)))
        v = v @ _rotation(rng).T
        s = rng.uniform(0.5, 1.0)
        meshes.append((_fit(v, s, 1.0, 3.0), f))
    return meshes, 256, 256, 10, 1e-4, GRAD_NAMES


def _soup1m(rng):
    v, f = _soup(rng, 1_000_000, -1.0, 1.0, 1.0, 3.0, 0.004)
    return [(v, f)], 1024, 1024, 1, 0.0, GRAD_NAMES


def _soups32(rng):
    meshes = []
    for _ in range(32):
        Fn = int(round(math.exp(rng.uniform(math.log(500.0), math.log(2e5)))))
        meshes.append(_soup(rng, Fn, -1.0, 1.0, 0.5, 4.0, 0.01, neg_frac=0.05))
    return meshes, 512, 512, 50, 1e-3, GRAD_NAMES


# name -> (builder, description). Index i uses geometry seed 1000+i, grad seed 2000+i.
CONFIGS = {
    "sphere64": (_sphere64, "1 icosphere L2 (320 tris), 64x64, K=1, blur=0"),
    "spheres8_137": (_spheres8, "8 icospheres L4 (5120 tris each), 137x137, K=8, blur=1e-4"),
    "hetero16_256": (_hetero16, "16 icospheres L3-6 (1280-81920 tris), 256x256, K=10, blur=1e-4"),
    "soup1m_1024": (_soup1m, "1,000,000-triangle soup, 1024x1024, K=1, blur=0"),
    "soups32_512": (_soups32, "32 soups, 500-200000 tris log-uniform, 512x512, K=50, blur=1e-3"),
}


# Reduced versions of the same recipes, small enough for a full-image oracle run
# in a few seconds while still spanning several tiles and a ragged tail.
def _small_hetero(rng):
    spheres = {L: icosphere(L) for L in (2, 3, 4)}
    meshes = []
    for _ in range(4):
        L = int(rng.integers(2, 5))
        base, f = spheres[L]
        v = base * (1.0 + rng.normal(0.0, 0.05, (base.shape[0], 1)))
        v = v @ _rotation(rng).T
        meshes.append((_fit(v, rng.uniform(0.5, 1.0), 1.0, 3.0), f))
    # an empty mesh in the middle of the batch
    meshes.insert(2, (np.zeros((0, 3)), np.zeros((0, 3), np.int64)))
    return meshes, 72, 56, 10, 1e-4, GRAD_NAMES


def _small_soup(rng):
    v, f = _soup(rng, 20_000, -1.0, 1.0, 1.0, 3.0, 0.01)
    return [(v, f)], 100, 130, 1, 0.0, GRAD_NAMES


def _small_soups(rng):
    meshes = []
    for _ in range(3):
        Fn = int(round(math.exp(rng.uniform(math.log(200.0), math.log(3000.0)))))
        meshes.append(_soup(rng, Fn, -1.0, 1.0, 0.5, 4.0, 0.03, neg_frac=0.05))
    return meshes, 40, 48, 50, 1e-3, GRAD_NAMES


SMALL_CONFIGS = {
    "small_hetero": _small_hetero,
    "small_soup": _small_soup,
    "small_soups": _small_soups,
}


def make_workload(name: str, seed: Optional[int] = None, grad_seed: Optional[int] = None) -> Workload:
    if name in CONFIGS:
        idx = list(CONFIGS).index(name)
        builder = CONFIGS[name][0]
    elif name in SMALL_CONFIGS:
        idx = 10 + list(SMALL_CONFIGS).index(name)
        builder = SMALL_CONFIGS[name]
    else:
        raise KeyError(f"unknown workload {name!r}")
    seed = 1000 + idx if seed is None else seed
    grad_seed = 2000 + idx if grad_seed is None else grad_seed
    rng = np.random.Generator(np.random.PCG64(seed))
    meshes, H, W, K, blur, grads = builder(rng)
    verts, faces, offsets = _pack(meshes)
    return Workload(name, verts, faces, offsets, H, W, K, float(np.float32(blur)), tuple(grads), seed, grad_seed)


def upstream_grads(w: Workload, seed: Optional[int] = None, which: Optional[Sequence[str]] = None):
    """Dense N(0,1) float32 upstream gradients over every slot (padding included).

    Returns a dict with keys 'zbuf' [N,H,W,K], 'bary' [N,H,W,K,3], 'dists'
    [N,H,W,K]; a gradient the workload does not drive is None."""
    rng = np.random.Generator(np.random.PCG64(w.grad_seed if seed is None else seed))
    which = w.grads if which is None else tuple(which)
    shape = (w.N, w.H, w.W, w.K)
    out = {}
    for g in GRAD_NAMES:
        if g in which:
            s = shape + ((3,) if g == "bary" else ())
            out[g] = rng.standard_normal(s, dtype=np.float32)
        else:
            out[g] = None
    return out


def sample_pixels(w: Workload, count: int, seed: int = 7) -> np.ndarray:
    """Sorted unique flat pixel ids (n*H*W + i*W + j): the four corners of every
    image plus `count` uniformly drawn pixels."""
    rng = np.random.Generator(np.random.PCG64(seed))
    HW = w.H * w.W
    corners = []
    for n in range(w.N):
        for (i, j) in ((0, 0), (0, w.W - 1), (w.H - 1, 0), (w.H - 1, w.W - 1)):
            corners.append(n * HW + i * w.W + j)
    drawn = rng.integers(0, w.pixels, count)
    return np.unique(np.concatenate([np.asarray(corners, np.int64), drawn.astype(np.int64)]))


def masked_upstream_grads(w: Workload, pixel_ids: np.ndarray, seed: Optional[int] = None):
    """N(0,1) upstream gradients on the given pixels only (all other slots are 0).

    Returned sparse: a dict of arrays shaped [len(pixel_ids), K] (or [.., K, 3]
    for 'bary'), or None for gradients the workload does not drive."""
    rng = np.random.Generator(np.random.PCG64((w.grad_seed if seed is None else seed) + 7919))
    S = len(pixel_ids)
    out = {}
    for g in GRAD_NAMES:
        if g in w.grads:
            s = (S, w.K) + ((3,) if g == "bary" else ())
            out[g] = rng.standard_normal(s, dtype=np.float32)
        else:
            out[g] = None
    return out


def face_colors(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Seeded per-face RGB colours in [0, 1) for the second stage, [F, 3] float32."""
    rng = np.random.Generator(np.random.PCG64((w.grad_seed if seed is None else seed) + 104729))
    return rng.random((w.F, 3), dtype=np.float32)


def blend_upstream_grads(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Dense N(0,1) float32 gradients of the blended RGBA image, [N, H, W, 4]."""
    rng = np.random.Generator(np.random.PCG64((w.grad_seed if seed is None else seed) + 130363))
    return rng.standard_normal((w.N, w.H, w.W, 4), dtype=np.float32)


def vert_offsets(w: Workload) -> np.ndarray:
    """[N+1] int64 vertex ranges of the meshes: mesh n owns vertices
    [vo[n], vo[n+1]) (the workloads pack each mesh's vertices together)."""
    vo = [0]
    for n in range(w.N):
        f = w.faces[w.offsets[n]:w.offsets[n + 1]]
        vo.append(max(vo[-1], int(f.max()) + 1) if f.size else vo[-1])
    vo[-1] = w.V
    return np.asarray(vo, np.int64)


def projection_inputs(w: Workload, seed: Optional[int] = None):
    """World-space vertices and per-mesh 4x4 cameras (row-major) whose
    projection (x/w, y/w, depth) gives back the workload's screen-space
    vertices up to rounding: each mesh gets a random rotation R, translation
    t and focal length f in [1.5, 2.5]; its screen vertices (x, y, z) are
    lifted to view space (x z / f, y z / f, z) and moved to world space by
    R^T (p - t). The camera is [[f R_0, f t_0], [f R_1, f t_1], [R_2, t_2],
    [R_2, t_2]].

    Returns (verts_world [V,3] float32, vert_offsets [N+1] int64,
    cameras [N,4,4] float32)."""
    rng = np.random.Generator(np.random.PCG64((w.seed if seed is None else seed) + 7919))
    vo = vert_offsets(w)
    world = np.zeros((w.V, 3), np.float64)
    cams = np.zeros((w.N, 4, 4), np.float64)
    for n in range(w.N):
        R = _rotation(rng)
        t = rng.normal(0.0, 1.0, 3)
        f = rng.uniform(1.5, 2.5)
        s = w.verts[vo[n]:vo[n + 1]].astype(np.float64)
        view = np.stack([s[:, 0] * s[:, 2] / f, s[:, 1] * s[:, 2] / f, s[:, 2]], axis=1)
        world[vo[n]:vo[n + 1]] = (view - t) @ R   # R^T (p - t), row vectors
        cams[n, 0, :3], cams[n, 0, 3] = f * R[0], f * t[0]
        cams[n, 1, :3], cams[n, 1, 3] = f * R[1], f * t[1]
        cams[n, 2, :3], cams[n, 2, 3] = R[2], t[2]
        cams[n, 3, :3], cams[n, 3, 3] = R[2], t[2]
    return world.astype(np.float32), vo, cams.astype(np.float32)


def projection_upstream_grads(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Dense N(0,1) float32 gradients of the projected vertices, [V, 3]."""
    rng = np.random.Generator(np.random.PCG64((w.grad_seed if seed is None else seed) + 15485863))
    return rng.standard_normal((w.V, 3), dtype=np.float32)


# ----------------------------------------------------------------------------
# point clouds
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class PointWorkload:
    name: str
    points: np.ndarray   # [P, 3] float32 (x, y NDC, z depth)
    offsets: np.ndarray  # [N + 1] int64: cloud n owns points [offsets[n], offsets[n+1])
    H: int
    W: int
    K: int
    radius: float        # a float32 value, NDC units
    seed: int
    grad_seed: int

    @property
    def N(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def P(self) -> int:
        return int(self.points.shape[0])

    @property
    def slots(self) -> int:
        return self.N * self.H * self.W * self.K

    @property
    def pixels(self) -> int:
        return self.N * self.H * self.W


def _points_from_meshes(mesh_name, H, W, K, radius):
    w = make_workload(mesh_name)
    return w.verts.copy(), vert_offsets(w), H, W, K, radius, w.seed, w.grad_seed


def _points_soup(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    clouds = []
    for n, P in enumerate((5000, 0, 3000)):
        p = np.empty((P, 3))
        p[:, 0] = rng.uniform(-1.1, 1.1, P)
        p[:, 1] = rng.uniform(-1.1, 1.1, P)
        p[:, 2] = rng.uniform(-0.5, 3.0, P)          # about 1 in 7 behind the camera
        if P:
            p[: P // 10] = p[P // 10: 2 * (P // 10)]   # exact duplicates: ties of (z) broken by index
            g = np.round(p[2 * (P // 10): 3 * (P // 10), :2] * 32) / 32
            p[2 * (P // 10): 3 * (P // 10), :2] = g  # on a dyadic grid: distances exact
        clouds.append(p)
    pts = np.concatenate(clouds).astype(np.float32)
    offs = np.concatenate([[0], np.cumsum([len(c) for c in clouds])]).astype(np.int64)
    return pts, offs, 64, 80, 5, 0.03125, seed, seed + 1000


# name -> builder; the clouds of the mesh workloads are their vertices
POINT_CONFIGS = {
    "points16_256": lambda: _points_from_meshes("hetero16_256", 256, 256, 10, 0.01),
    "points_small": lambda: _points_from_meshes("small_hetero", 72, 56, 8, 0.03),
    "points_soup": lambda: _points_soup(3100),
}


def make_point_workload(name: str) -> PointWorkload:
    pts, offs, H, W, K, radius, seed, grad_seed = POINT_CONFIGS[name]()
    return PointWorkload(name, pts, offs, H, W, K, float(np.float32(radius)), seed, grad_seed)


def point_upstream_grads(w: PointWorkload, seed: Optional[int] = None):
    """Dense N(0,1) float32 gradients of zbuf and dists, each [N,H,W,K]."""
    rng = np.random.Generator(np.random.PCG64((w.grad_seed if seed is None else seed) + 32452843))
    shape = (w.N, w.H, w.W, w.K)
    return {"zbuf": rng.standard_normal(shape, dtype=np.float32),
            "dists": rng.standard_normal(shape, dtype=np.float32)}

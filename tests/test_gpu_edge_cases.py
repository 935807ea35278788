"""GPU path against the oracle on edge cases: empty meshes and batches, K
beyond the candidate count, culled and degenerate faces, exact depth ties,
pixel centres on shared edges, thin and one-pixel images, K = 1 and K = 64,
a blur radius covering the image, off-screen faces, one face over every bin,
thousands of faces in one bin, heavy bins split into quarter items, hundreds
of faces each covering every pixel (whole and split bins, K up to 64), subnormal depths,
faces using another mesh's vertices, the largest image side, hundreds of
small meshes, near-degenerate slivers (tiny non-zero doubled area), faces
whose arithmetic meets NaN or overflow, invalid vertex indices, and the
hand-worked cases; every case also through the
backward pass."""

import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import GpuCase, host, require_gpu, say, to_dev
from parity import assert_forward_parity, compare_forward, oracle_excuse, rel_l2

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


@pytest.fixture(scope="module")
def dmr():
    return require_gpu()


def _check(verts, faces, offsets, H, W, K, blur, expect_flags=0):
    verts = np.asarray(verts, np.float32).reshape(-1, 3)
    faces = np.asarray(faces, np.int64).reshape(-1, 3)
    offsets = np.asarray(offsets, np.int64)
    g = GpuCase(verts, faces, offsets, H, W, K, blur)
    got = host(g.forward())
    ref = oracle.rasterize(verts, faces, offsets, H, W, K, blur)
    rep = compare_forward(ref, got, K, excuse=oracle_excuse(oracle, verts, faces, offsets, H, W, blur))
    assert_forward_parity(rep, max_excused_frac=0.0)
    assert g.stats()["flags"] == expect_flags
    return got, ref


def _soup(seed, F, lo=-1.0, hi=1.0, sigma=0.05, zlo=0.5, zhi=3.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = np.stack([rng.uniform(lo, hi, F), rng.uniform(lo, hi, F), rng.uniform(zlo, zhi, F)], 1)
    v = (c[:, None, :] + rng.normal(0, sigma, (F, 3, 3))).reshape(-1, 3)
    return v.astype(np.float32), np.arange(3 * F).reshape(F, 3)


CASES = {}


def case(fn):
    CASES[fn.__name__] = fn
    return fn


@case
def all_meshes_empty():
    return np.zeros((0, 3)), np.zeros((0, 3)), [0, 0, 0, 0], 8, 8, 3, 0.0


@case
def empty_mesh_between():
    v, f = _soup(1, 40)
    return v, f, [0, 20, 20, 40], 24, 24, 4, 1e-3


@case
def k_beyond_candidates_k64():
    v, f = _soup(2, 30, sigma=0.3)
    return v, f, [0, 30], 20, 20, 64, 1e-3


@case
def all_culled():
    v, f = _soup(3, 50, zlo=-2.0, zhi=-0.1, sigma=0.02)
    return v, f, [0, 50], 16, 16, 2, 1e-3


@case
def straddling_depth():
    v, f = _soup(4, 60, zlo=-0.2, zhi=0.2, sigma=0.3)
    return v, f, [0, 60], 32, 32, 3, 0.0


@case
def degenerate_mixed():
    v, f = _soup(5, 30)
    v = v.reshape(30, 3, 3)
    v[::3, 2, :2] = 0.5 * (v[::3, 0, :2] + v[::3, 1, :2])  # collinear
    v[1::5, 1] = v[1::5, 0]  # repeated vertex
    return v.reshape(-1, 3), f, [0, 30], 32, 32, 2, 1e-2


@case
def coincident_faces():
    v, f = _soup(6, 10, sigma=0.3)
    f = np.concatenate([f, f, f[::-1]])
    return v, f, [0, 30], 24, 24, 5, 1e-3


@case
def shared_edges_through_centres():
    # a square split along its diagonal; with 8x8 pixels the centres +-k/8
    # lie exactly on the diagonal x = y
    v = [[-0.75, -0.75, 1], [0.75, -0.75, 1], [0.75, 0.75, 1], [-0.75, 0.75, 1]]
    f = [[0, 1, 2], [0, 2, 3]]
    return v, f, [0, 2], 8, 8, 2, 0.0


@case
def thin_images_h1():
    v, f = _soup(7, 50, sigma=0.2)
    return v, f, [0, 50], 1, 37, 3, 1e-3


@case
def thin_images_w1():
    v, f = _soup(8, 50, sigma=0.2)
    return v, f, [0, 50], 45, 1, 3, 1e-3


@case
def one_pixel():
    v, f = _soup(9, 20, sigma=0.5)
    return v, f, [0, 20], 1, 1, 4, 0.0


@case
def k1_zbuffer():
    v, f = _soup(10, 200)
    return v, f, [0, 200], 40, 33, 1, 0.0


@case
def blur_covers_image():
    v, f = _soup(11, 12, sigma=0.02)
    return v, f, [0, 12], 12, 12, 16, 8.0


@case
def off_screen_faces():
    v, f = _soup(12, 60, lo=1.2, hi=3.0)
    v2, f2 = _soup(13, 20)
    v = np.concatenate([v, v2])
    f = np.concatenate([f, f2 + 180])
    return v, f, [0, 80], 20, 20, 2, 1e-3


@case
def one_face_over_all_bins():
    v = [[-3, -3, 2], [5, -3, 1], [-3, 5, 3]]
    v2, f2 = _soup(14, 40)
    v = np.concatenate([np.asarray(v, np.float32), v2])
    f = np.concatenate([[[0, 1, 2]], f2 + 3])
    return v, f, [0, 41], 150, 170, 3, 1e-4


@case
def thousands_in_one_bin():
    v, f = _soup(15, 5000, lo=-0.95, hi=-0.9, sigma=0.01)
    return v, f, [0, 5000], 64, 64, 8, 1e-4


@case
def dense_bins_split_into_quarters():
    # about 3000 faces over one and a half bins: the heavy bins are worked
    # as four 8x8 quarter items with four lanes per pixel
    v, f = _soup(18, 3000, lo=-1.0, hi=-0.4, sigma=0.02)
    return v, f, [0, 3000], 40, 56, 10, 1e-4


@case
def dense_split_bins_on_ragged_edge():
    # split bins in the last bin row and column, partly outside the image
    v, f = _soup(19, 2500, lo=0.75, hi=1.0, sigma=0.02)
    return v, f, [0, 2500], 37, 45, 16, 5e-4


def _covering(seed, F):
    """F large triangles that each cover the whole image, with depths spread
    over [0.5, 3] per vertex, so that depth bounds prune little."""
    rng = np.random.Generator(np.random.PCG64(seed))
    base = np.array([[-3.0, -3.0], [5.0, -3.0], [-3.0, 5.0]])
    xy = base[None] + rng.uniform(-0.3, 0.3, (F, 3, 2))
    z = rng.uniform(0.5, 3.0, (F, 3, 1))
    v = np.concatenate([xy, z], 2).reshape(-1, 3)
    return v.astype(np.float32), np.arange(3 * F).reshape(F, 3)


@case
def all_faces_cover_every_pixel():
    # every pixel has every staged face as a candidate: 256 pairs per pixel
    # per round, many pair windows per round
    v, f = _covering(20, 700)
    return v, f, [0, 700], 32, 32, 12, 1e-3


@case
def all_faces_cover_a_split_bin():
    # 2,400 faces over one bin: four quarter items, four owners per pixel,
    # each with 64 candidates per round
    v, f = _covering(21, 2400)
    return v, f, [0, 2400], 16, 16, 10, 1e-4


@case
def all_faces_cover_every_pixel_k32():
    # dense rounds of a long list with K = 32: every owner has 256 candidate
    # pairs per round, so the rounds go to per-owner loops
    v, f = _covering(23, 500)
    return v, f, [0, 500], 24, 40, 32, 1e-3


@case
def all_faces_cover_every_pixel_k64():
    v, f = _covering(24, 400)
    return v, f, [0, 400], 20, 20, 64, 1e-3


@case
def all_faces_cover_a_split_bin_k16():
    # quarter items whose four owners per pixel each have 64 candidates per
    # round: dense rounds in per-owner loops on the quarter's own face word
    v, f = _covering(25, 2400)
    return v, f, [0, 2400], 16, 16, 16, 1e-4


@case
def all_faces_cover_a_split_bin_k1():
    # quarter items at K = 1, whose rounds always take the per-owner loops:
    # each owner keeps its own nearest face and the quad's are merged
    v, f = _covering(26, 2400)
    return v, f, [0, 2400], 16, 16, 1, 0.0


@case
def all_faces_cover_a_split_bin_k2():
    v, f = _covering(27, 2200)
    return v, f, [0, 2200], 16, 16, 2, 1e-4


@case
def tiny_positive_depths():
    # depths down to binary32 subnormals: their keys read as binary64 are
    # subnormal too, and must still order exactly
    rng = np.random.Generator(np.random.PCG64(22))
    v, f = _soup(22, 300, sigma=0.08)
    v[:, 2] = (rng.uniform(1.0, 2.0, len(v)) * 10.0 ** rng.integers(-44, -36, len(v))).astype(np.float32)
    return v, f, [0, 300], 24, 20, 8, 1e-3


@case
def faces_use_other_meshes_vertices():
    v, f = _soup(16, 40)
    f = f.copy()
    f[30:40] = f[0:10]  # mesh 1 reuses mesh 0's vertices
    return v, f, [0, 20, 40], 16, 16, 3, 1e-3


@case
def large_coordinates():
    v = [[-50, -40, 2], [60, -10, 1], [0, 70, 3], [-0.5, -0.5, 1], [0.5, -0.4, 1], [0.1, 0.6, 1]]
    return v, [[0, 1, 2], [3, 4, 5]], [0, 2], 30, 30, 2, 1e-3


@case
def max_width_image():
    # the largest image side: 2048 bins per row, faces spread along it
    rng = np.random.Generator(np.random.PCG64(20))
    x = rng.uniform(-1.0, 1.0, 60)
    z = rng.uniform(1.0, 2.0, 60)
    w = rng.uniform(1e-4, 4e-4, 60)   # 2 to 6 pixels wide
    v = np.stack([np.stack([x - w, np.full(60, -0.9), z], 1), np.stack([x + w, np.full(60, -0.8), z], 1),
                  np.stack([x, np.full(60, 0.9), z + 0.1], 1)], 1).reshape(-1, 3).astype(np.float32)
    return v, np.arange(180).reshape(60, 3), [0, 60], 2, 32767, 3, 1e-9


@case
def many_small_meshes():
    # 600 meshes of 0-3 faces: setup workgroups span many meshes, so most
    # bin counts take the global path
    rng = np.random.Generator(np.random.PCG64(21))
    sizes = rng.integers(0, 4, 600)
    v, f = _soup(22, int(sizes.sum()), sigma=0.3)
    return v, f, np.concatenate([[0], np.cumsum(sizes)]), 8, 8, 2, 1e-2


def _slivers(seed, F):
    """Near-degenerate slivers: v2 continues the segment v0 -> v1 to twice
    its length and is then moved by a few units in the last place, so the
    binary32 doubled area A is tiny but non-zero (1e-9 down to about 1e-13;
    v0 is drawn at scales 1e-3 to 0.3 around the image centre, where the
    last place of a coordinate is small). Their raw barycentrics at a pixel
    are edge functions of O(0.1) size divided by A: the rounding noise of the
    edge functions can give every barycentric a positive sign at pixel
    centres far outside the sliver, where only the bounding-box clause of the
    inside test keeps the face out."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f32 = np.float32
    n = 8 * F
    scale = 10.0 ** rng.uniform(-3.0, -0.5, (n, 1))
    a = (scale * rng.uniform(-1.0, 1.0, (n, 2))).astype(f32)
    t = rng.uniform(0.0, 2.0 * np.pi, n)
    d = (rng.uniform(0.02, 0.4, (n, 1)) * np.stack([np.cos(t), np.sin(t)], 1)).astype(f32)
    b = (a + d).astype(f32)
    c = (a + f32(2) * d).astype(f32)
    nudge = rng.integers(-3, 4, (n, 2)).astype(f32)
    c = (c + nudge * np.spacing(np.abs(c)).astype(f32)).astype(f32)
    x0, y0, x1, y1, x2, y2 = a[:, 0], a[:, 1], b[:, 0], b[:, 1], c[:, 0], c[:, 1]
    A = (x1 - x0) * (y2 - y0) - (y1 - y0) * (x2 - x0)   # binary32, in the conventions' order
    assert A.dtype == np.float32
    keep = np.nonzero((np.abs(A) > 0) & (np.abs(A) < 1e-9))[0][:F]
    assert len(keep) == F and np.abs(A[keep]).min() < 1e-11 and (np.abs(A[keep]) < 1e-10).sum() > F // 10
    z = rng.uniform(1.0, 3.0, (F, 3)).astype(f32)
    v = np.stack([np.concatenate([a[keep], z[:, :1]], 1), np.concatenate([b[keep], z[:, 1:2]], 1),
                  np.concatenate([c[keep], z[:, 2:]], 1)], 1).astype(f32)
    return v.reshape(-1, 3), np.arange(3 * F).reshape(F, 3)


@case
def near_degenerate_slivers():
    v, f = _slivers(23, 400)
    return v, f, [0, 400], 64, 64, 3, 0.0


@case
def near_degenerate_slivers_blur():
    v, f = _slivers(24, 400)
    return v, f, [0, 400], 48, 56, 4, 1e-4


@case
def faces_on_the_nan_path():
    # ordinary faces sharing bins with faces whose per-pixel arithmetic can
    # meet NaN or overflow: coordinates of 1e20 and 1e30, a doubled area
    # below 2^-128 (1/A overflows) and an edge too short to square (its
    # inverse squared length overflows); their rounds take the exact
    # NaN-propagating evaluation, the others the median clamps
    v, f = _soup(25, 120, sigma=0.1)
    extra = np.array([
        [-1e20, -0.5, 1.0], [1e20, -0.4, 2.0], [0.0, 1e20, 1.5],          # huge coordinates
        [-0.3, -1e30, 1.2], [0.4, 0.2, 1.1], [-0.2, 0.3, 1.3],
        [0.0, 0.0, 1.0], [1e-20, 0.0, 1.0], [0.0, 1e-19, 1.0],           # A = 1e-39: 1/A overflows
        [1e-22, 0.3, 0.9], [2e-22, 0.3, 0.9], [0.6, -0.6, 2.0],         # |edge|^2 = 1e-44: 1/|edge|^2 overflows
    ], np.float32)
    fe = np.arange(len(v), len(v) + 12).reshape(4, 3)
    return (np.concatenate([v, extra]), np.concatenate([f, fe]), [0, 124], 40, 48, 4, 2e-3)


@pytest.mark.parametrize("name", list(CASES))
def test_edge_case(dmr, name):
    say(f"[gpu] edge case {name}")
    _check(*CASES[name]())


@pytest.mark.parametrize("name", list(CASES))
def test_edge_case_backward(dmr, name):
    # the same inputs through the backward pass, with seeded N(0, 1) upstream
    # gradients on every slot (the padding's must be ignored by both sides)
    verts, faces, offsets, H, W, K, blur = CASES[name]()
    verts = np.asarray(verts, np.float32).reshape(-1, 3)
    faces = np.asarray(faces, np.int64).reshape(-1, 3)
    offsets = np.asarray(offsets, np.int64)
    say(f"[gpu] edge case backward {name}")
    g = GpuCase(verts, faces, offsets, H, W, K, blur)
    p2f = g.forward()[0]
    ref_p2f = oracle.rasterize(verts, faces, offsets, H, W, K, blur)[0]
    assert np.array_equal(p2f.cpu().numpy(), ref_p2f)
    rng = np.random.Generator(np.random.PCG64(7000 + list(CASES).index(name)))
    shape = ref_p2f.shape
    gz = rng.standard_normal(shape).astype(np.float32)
    gb = rng.standard_normal(shape + (3,)).astype(np.float32)
    gd = rng.standard_normal(shape).astype(np.float32)
    gv = g.backward(p2f, to_dev(gz), to_dev(gb), to_dev(gd)).cpu().numpy()
    ref = oracle.backward(verts, faces, offsets, H, W, K, blur, ref_p2f, gz, gb, gd)
    if not np.any(ref_p2f >= 0):
        assert not np.any(gv)
    else:
        # faces whose partials overflow or meet NaN give non-finite vertex
        # gradients on both sides (which ones does not depend on the order
        # of the sums); the finite ones are compared
        fin = np.isfinite(ref.astype(np.float32))
        assert np.array_equal(fin, np.isfinite(gv))
        err = rel_l2(gv[fin], ref[fin])
        say(f"  rel L2 = {err:.2e}  |ref| = {np.linalg.norm(ref[fin]):.3e}  non-finite {int((~fin).sum())}")
        assert err <= 1e-4


def test_invalid_vertex_index_is_flagged(dmr):
    v, f = _soup(17, 20)
    f = f.copy()
    f[3, 1] = 10_000
    f[7, 0] = -5
    say("[gpu] invalid vertex indices")
    _check(v, f, [0, 20], 16, 16, 2, 1e-3, expect_flags=1)


def test_hand_cases_on_gpu(dmr):
    with open(GOLDEN) as fh:
        data = json.load(fh)
    import test_oracle_golden as T1

    for c in data["cases"]:
        say(f"[gpu] hand case {c['name']}")
        v, f, o = T1._inputs(c)
        g = GpuCase(v, f, o, c["H"], c["W"], c["K"], c["blur"])
        got = host(g.forward())
        for a, b in zip(got, T1._expected(c, np.float32)):
            assert np.array_equal(a, b), c["name"]

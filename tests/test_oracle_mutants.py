"""The oracle's pins are sharp: each plausible mistake planted in a copy of the
oracle source (a flipped comparison, a dropped term, a transposed operand, a
wrong index or sign) must make at least one pin fail.

The planted copies are built in a temporary directory on the CPU; the real
oracle is never modified.
"""

import json
import os
import shutil

import numpy as np
import pytest

import test_oracle_exact as T2
import test_oracle_fd as T4
import test_oracle_settings as T5
from exact_raster import exact_rasterize
from parity import compare_forward, exact_excuse

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")

# (name, original text, planted text)
MUTANTS = [
    ("inside_not_strict", "(s->b[0] > (R)0) && (s->b[1] > (R)0)", "(s->b[0] >= (R)0) && (s->b[1] >= (R)0)"),
    ("blur_not_strict", "s->d2 < blur", "s->d2 <= blur"),
    ("tie_break_reversed", "if (a->face < b->face) return -1;", "if (a->face < b->face) return 1;"),
    ("z_zero_kept", "if (!(s->zp > (R)0)) return 0;", "if (s->zp < (R)0) return 0;"),
    ("edge_function_sign", "s->w[1] = s->dx[2] * s->dy[0] - s->dy[2] * s->dx[0];",
     "s->w[1] = s->dy[2] * s->dx[0] - s->dx[2] * s->dy[0];"),
    ("distance_transposed", "s->ry[e] = qy - t * uy;", "s->ry[e] = qy - t * ux;"),
    ("no_renormalisation", "s->bh[k] = s->c[k] * s->invS;", "s->bh[k] = s->c[k];"),
    ("no_lower_clip", "if (c < (R)0) c = (R)0;", ""),
    ("no_t_clamp", "if (t > (R)1) t = (R)1;", ""),
    ("pixel_axis_flipped", "return (R)(2 * j + 1) / (R)W - (R)1;", "return (R)1 - (R)(2 * j + 1) / (R)W;"),
    ("depth_wrong_vertex", "s->bh[1] * s->z[1]) + s->bh[2] * s->z[2]", "s->bh[1] * s->z[2]) + s->bh[2] * s->z[2]"),
    ("bwd_edge_partial_index", "gx[1] += gw[0] * s.dy[2];", "gx[1] += gw[0] * s.dy[1];"),
    ("bwd_area_sign", "R gA = -((gb[0]", "R gA = ((gb[0]"),
    ("bwd_clip_gate_dropped", "(s.b[c] > (R)0 && s.b[c] < (R)1) ? gc : (R)0", "gc"),
    ("bwd_dist_weight", "R ga = gd2 * (R)-2 * ((R)1 - t);", "R ga = gd2 * (R)-2 * t;"),
    ("bwd_inside_sign", "R gd2 = s.inside ? -gd : gd;", "R gd2 = gd;"),
    ("bwd_renorm_dot_dropped", "gc = (gbh[c] - dot) * s.invS;", "gc = gbh[c] * s.invS;"),
    ("bwd_depth_grad", "gzv[c] = gz * s.bh[c];", "gzv[c] = gz * s.c[c];"),
    # settings (perspective-correct, back-face culling, unclipped barycentrics)
    ("persp_weight_index", "s->n[k] = (s->c[k] * s->z[(k + 1) % 3]) * s->z[(k + 2) % 3];",
     "s->n[k] = (s->c[k] * s->z[k]) * s->z[(k + 2) % 3];"),
    ("persp_depth_guard_dropped",
     "if ((settings & ORACLE_PERSPECTIVE) && !(s->z[0] > (R)0 && s->z[1] > (R)0 && s->z[2] > (R)0)) return 0;", ""),
    ("cull_sign", "(settings & ORACLE_CULL_BACK) && s->A > (R)0", "(settings & ORACLE_CULL_BACK) && s->A < (R)0"),
    ("raw_persp_from_clipped", "s->nr[k] = (s->b[k] * s->z[(k + 1) % 3])", "s->nr[k] = (s->c[k] * s->z[(k + 1) % 3])"),
    ("raw_returns_clipped", "for (int k = 0; k < 3; ++k) s->out[k] = s->b[k];", ""),
    ("bwd_persp_dot_dropped", "R gn = (gbh[c] - dot) * s.invD;", "R gn = gbh[c] * s.invD;"),
    ("bwd_persp_dz_index", "gzv[c1] += gn * (s.c[c] * s.z[c2]);", "gzv[c1] += gn * (s.c[c] * s.z[c1]);"),
    ("bwd_raw_grad_dropped", "for (int c = 0; c < 3; ++c) gb[c] += gout[c];", ""),
    ("bwd_raw_persp_dz_index", "gzv[c2] += gn * (s.b[c] * s.z[c1]);", "gzv[c2] += gn * (s.b[c] * s.z[c2]);"),
]


def _golden_ok(oracle, lib):
    with open(GOLDEN) as fh:
        data = json.load(fh)
    import test_oracle_golden as T1

    for case in data["cases"]:
        v, f, o = T1._inputs(case)
        got = oracle.rasterize(v, f, o, case["H"], case["W"], case["K"], case["blur"], lib_path=lib)
        for g, e in zip(got, T1._expected(case, np.float32)):
            if not np.array_equal(g, e):
                return False
    cases = {c["name"]: c for c in data["cases"]}
    for bc in data["backward_cases"]:
        case = cases[bc["case"]]
        v, f, o = T1._inputs(case)
        H, W, K = case["H"], case["W"], case["K"]
        p2f = oracle.rasterize(v, f, o, H, W, K, case["blur"], lib_path=lib)[0]
        px = bc["pixel"]
        for g in bc["grads"]:
            gz = np.zeros((1, H, W, K), np.float32)
            gb = np.zeros((1, H, W, K, 3), np.float32)
            gd = np.zeros((1, H, W, K), np.float32)
            gz[0, px["i"], px["j"], px["slot"]] = g["gz"]
            gb[0, px["i"], px["j"], px["slot"]] = g["gbary"]
            gd[0, px["i"], px["j"], px["slot"]] = g["gd"]
            got = oracle.backward(v, f, o, H, W, K, case["blur"], p2f, gz, gb, gd, lib_path=lib)
            if not np.array_equal(got, np.asarray(g["grad_verts"], np.float64)):
                return False
    return True


def _exact_ok(oracle, lib):
    for seed in range(12):
        v, f, o, H, W, K, blur = T2._case(seed)
        exact, details = exact_rasterize(v, f, o, H, W, K, blur)
        got = oracle.rasterize(v, f, o, H, W, K, blur, lib_path=lib)
        rep = compare_forward(exact, got, K, atol=2e-6, excuse=exact_excuse(details, len(o) - 1, H, W, blur))
        if rep["unexcused"] or not rep["values_ok"] or not rep["padding_ok"]:
            return False
    return True


def _fd_ok(oracle, lib):
    H = W = T4.H
    for seed in range(6):
        v, f, o, K, blur, g = T4._scene(seed)
        p2f = oracle.rasterize(v, f, o, H, W, K, blur, precision="f64", lib_path=lib)[0]
        grad = oracle.backward(v, f, o, H, W, K, blur, p2f, g["zbuf"].astype(np.float32),
                               g["bary"].astype(np.float32), g["dists"].astype(np.float32),
                               precision="f64", lib_path=lib)
        g32 = {k: a.astype(np.float32).astype(np.float64) for k, a in g.items()}

        def loss(vv):
            out = oracle.rasterize(vv, f, o, H, W, K, blur, precision="f64", with_state=True, lib_path=lib)
            return ((g32["zbuf"] * out[1]).sum() + (g32["bary"] * out[2]).sum()
                    + (g32["dists"] * out[3]).sum()), out[0], out[4]

        _, p0, s0 = loss(v)
        for vi in np.unique(f):
            for c in range(3):
                vp, vm = v.copy(), v.copy()
                vp[vi, c] += T4.STEP
                vm[vi, c] -= T4.STEP
                Lp, pp, sp = loss(vp)
                Lm, pm, sm = loss(vm)
                if not (np.array_equal(pp, p0) and np.array_equal(pm, p0)
                        and np.array_equal(sp, s0) and np.array_equal(sm, s0)):
                    continue
                fd = (Lp - Lm) / (2 * T4.STEP)
                if abs(fd - grad[vi, c]) > 1e-5 * (1 + abs(grad[vi, c])):
                    return False
    return True


class _Bound:
    """The oracle module with its calls directed to one built library."""

    def __init__(self, oracle, lib):
        self._oracle, self._lib = oracle, lib

    def rasterize(self, *args, **kw):
        return self._oracle.rasterize(*args, lib_path=self._lib, **kw)

    def backward(self, *args, **kw):
        return self._oracle.backward(*args, lib_path=self._lib, **kw)


def _settings_ok(oracle, lib):
    b = _Bound(oracle, lib)
    checks = [lambda: T5.test_perspective_matches_reciprocal_form(b, 0),
              lambda: T5.test_perspective_skips_faces_behind_the_camera(b),
              lambda: T5.test_culling_equals_degenerate_back_faces(b, 3),
              lambda: T5.test_culling_keeps_the_first_hit_of_closed_meshes(b),
              lambda: T5.test_unclipped_barycentrics(b, 5)]
    for name in T5.SETTINGS:
        for seed in range(4):
            checks.append(lambda name=name, seed=seed: T5.test_backward_matches_finite_differences(b, name, seed))
    for check in checks:
        try:
            check()
        except AssertionError:
            return False
    return True


def test_unmutated_copy_passes(oracle_mod, tmp_path):
    lib = oracle_mod.build(out_path=str(tmp_path / "lib.so"))
    assert _golden_ok(oracle_mod, lib) and _exact_ok(oracle_mod, lib) and _fd_ok(oracle_mod, lib)
    assert _settings_ok(oracle_mod, lib)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle_mod, tmp_path, mutant):
    name, old, new = mutant
    for fn in ("raster_oracle.c", "raster_oracle_impl.h"):
        shutil.copy(os.path.join(ORACLE_DIR, fn), tmp_path / fn)
    impl = tmp_path / "raster_oracle_impl.h"
    src = impl.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    impl.write_text(src.replace(old, new))
    lib = oracle_mod.build(out_path=str(tmp_path / "lib.so"), source_dir=str(tmp_path))
    caught = ((not _golden_ok(oracle_mod, lib)) or (not _exact_ok(oracle_mod, lib)) or (not _fd_ok(oracle_mod, lib))
              or (not _settings_ok(oracle_mod, lib)))
    assert caught, f"planted mistake {name} passed every pin"

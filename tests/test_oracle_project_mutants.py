"""The projection oracle's pins are sharp: each plausible mistake planted in
a copy of oracle/project.py (a wrong divisor or homogeneous coordinate, a
transposed camera, meshes given the wrong camera, a sign, power or index in
the backward pass, and in the error bounds that set the GPU tolerances a
dropped or shrunk term or an inflated bound) must make at least one pin of
test_oracle_project.py fail. The planted copies are imported from a
temporary directory; the real oracle is never modified."""

import importlib.util
import inspect
import os

import numpy as np
import pytest

import test_oracle_project as T

PROJECT_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "project.py")

FWD = "np.stack([h[:, 0] / h[:, 3], h[:, 1] / h[:, 3], h[:, 2]], axis=1)"
GH = "gh = np.stack([g[:, 0] / h[:, 3], g[:, 1] / h[:, 3], g[:, 2],"

# (name, original text, planted text, which occurrence of the original: 0 = first)
MUTANTS = [
    ("x_divides_by_depth", FWD, "np.stack([h[:, 0] / h[:, 2], h[:, 1] / h[:, 3], h[:, 2]], axis=1)", 0),
    ("z_divided", FWD, "np.stack([h[:, 0] / h[:, 3], h[:, 1] / h[:, 3], h[:, 2] / h[:, 3]], axis=1)", 0),
    ("homogeneous_zero_fwd", "np.ones((X.shape[0], 1))", "np.zeros((X.shape[0], 1))", 0),
    ("homogeneous_zero_bwd", "np.ones((X.shape[0], 1))", "np.zeros((X.shape[0], 1))", 1),
    ("camera_transposed", 'h = np.einsum("vrc,vc->vr", M[mesh], Xh)', 'h = np.einsum("vcr,vc->vr", M[mesh], Xh)', 0),
    ("mesh_cameras_reversed", "np.repeat(np.arange(len(off) - 1), np.diff(off))[:V]",
     "np.repeat(np.arange(len(off) - 1)[::-1], np.diff(off))[:V]", 0),
    ("bwd_h3_sign", "-(g[:, 0] * h[:, 0] + g[:, 1] * h[:, 1]) / (h[:, 3] * h[:, 3])",
     "(g[:, 0] * h[:, 0] + g[:, 1] * h[:, 1]) / (h[:, 3] * h[:, 3])", 0),
    ("bwd_h3_power", "/ (h[:, 3] * h[:, 3])], axis=1)", "/ h[:, 3]], axis=1)", 0),
    ("bwd_gh1_uses_g0", GH, "gh = np.stack([g[:, 0] / h[:, 3], g[:, 0] / h[:, 3], g[:, 2],", 0),
    ("bwd_vertex_transposed", 'gX = np.einsum("vrc,vr->vc", M[mesh][:, :, :3], gh)',
     'gX = np.einsum("vcr,vr->vc", M[mesh][:, :3, :3], gh[:, :3])', 0),
    ("bwd_camera_outer_transposed", "np.add.at(gM, mesh, gh[:, :, None] * Xh[:, None, :])",
     "np.add.at(gM, mesh, Xh[:, :, None] * gh[:, None, :])", 0),
    ("bwd_camera_to_first_mesh", "np.add.at(gM, mesh, gh", "np.add.at(gM, 0 * mesh, gh", 0),
    ("fwd_bound_gamma_small", "eh = 4 * u * a / (1 - 4 * u)", "eh = u * a / (1 - 4 * u)", 0),
    ("fwd_bound_quotient_rounding_dropped",
     "e0 = (eh[:, 0] + np.abs(q0) * eh[:, 3]) / np.abs(h[:, 3]) + u * np.abs(q0)",
     "e0 = (eh[:, 0] + np.abs(q0) * eh[:, 3]) / np.abs(h[:, 3])", 0),
    ("fwd_bound_divisor_error_dropped", "e1 = (eh[:, 1] + np.abs(q1) * eh[:, 3])", "e1 = (eh[:, 1])", 0),
    ("fwd_bound_inflated", "return np.stack([e0, e1, eh[:, 2]], axis=1)",
     "return 8.0 * np.stack([e0, e1, eh[:, 2]], axis=1)", 0),
    ("bwd_bound_inflated", "return 2 * bound_v, 2 * bound_m", "return 16 * bound_v, 2 * bound_m", 0),
    ("bwd_bound_camera_inflated", "return 2 * bound_v, 2 * bound_m", "return 2 * bound_v, 16 * bound_m", 0),
    ("bwd_bound_product_rounding_dropped", "dgh + g4 * gh)", "dgh)", 0),
    ("bwd_bound_sum_depth_dropped", "bound_m += (depth * u)[:, None, None] * sum_abs",
     "bound_m += 0.0 * sum_abs", 0),
    ("bwd_bound_h3_error_dropped", "g[:, 0] * eh[:, 3] / ah3 ** 2 + u * gh[:, 0]", "u * gh[:, 0]", 0),
]

PIN_NAMES = [n for n, f in inspect.getmembers(T, inspect.isfunction) if n.startswith("test_")]
ARGS = {"test_workload_cameras_give_back_the_screen_vertices": [("small_hetero",)]}


def _plant(tmp_path, name, orig, new, which):
    src = open(PROJECT_SRC).read()
    at = -1
    for _ in range(which + 1):
        at = src.index(orig, at + 1)
    src = src[:at] + new + src[at + len(orig):]
    path = tmp_path / f"project_{name}.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(f"project_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pins_pass(mod, monkeypatch):
    for fn in ("project_forward", "project_backward", "project_forward_error_bound", "project_backward_error_bound"):
        monkeypatch.setattr(T, fn, getattr(mod, fn))
    for name in PIN_NAMES:
        for args in ARGS.get(name, [()]):
            try:
                with np.errstate(all="ignore"):
                    getattr(T, name)(*args)
            except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError, IndexError):
                return False
    return True


def test_pins_pass_on_the_real_oracle(monkeypatch):
    import oracle.project as real

    assert _pins_pass(real, monkeypatch)


@pytest.mark.parametrize("name,orig,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, orig, new, which):
    mod = _plant(tmp_path, name, orig, new, which)
    assert not _pins_pass(mod, monkeypatch), f"planted mistake {name} passes every pin"

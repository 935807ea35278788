"""The point-cloud oracle's pins are sharp: each plausible mistake planted in
a copy of oracle/points.py (a shifted pixel centre, a non-strict or
unsquared radius, a dropped depth test, a wrong order or tie-break, a local
index, a transposed coordinate, a wrong output, a sign or factor in the
backward pass, padding slots counted) must make at least one pin of
test_oracle_points.py fail. The planted copies are imported from a temporary
directory; the real oracle is never modified."""

import importlib.util
import inspect
import os
import sys

import numpy as np
import pytest

import test_oracle_points as T

POINTS_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "points.py")

# (name, original text, planted text, which occurrence of the original: 0 = first)
MUTANTS = [
    ("centre_shift", "return (np.asarray(2 * j + 1, dt) / dt(n)) - dt(1)",
     "return (np.asarray(2 * j, dt) / dt(n)) - dt(1)", 0),
    ("radius_not_strict", "cand = (d2 < r2) & (q[None, :, 2] > 0)", "cand = (d2 <= r2) & (q[None, :, 2] > 0)", 0),
    ("behind_camera_kept", "cand = (d2 < r2) & (q[None, :, 2] > 0)", "cand = (d2 < r2)", 0),
    ("radius_not_squared", "r2 = dt(radius) * dt(radius)", "r2 = dt(radius)", 0),
    ("tie_by_descending_index", "order = np.lexsort((c, q[c, 2]))[:K]", "order = np.lexsort((-c, q[c, 2]))[:K]", 0),
    ("order_by_distance", "order = np.lexsort((c, q[c, 2]))[:K]", "order = np.lexsort((c, d2[a, c]))[:K]", 0),
    ("one_slot_short", "order = np.lexsort((c, q[c, 2]))[:K]", "order = np.lexsort((c, q[c, 2]))[:max(K - 1, 1)]", 0),
    ("local_index", "idx[row, :m] = lo + c", "idx[row, :m] = c", 0),
    ("dx_uses_y", "dx = px - q[None, :, 0]", "dx = px - q[None, :, 1]", 0),
    ("rows_from_columns", "py = ys[rem // W][:, None]", "py = ys[(rem % W) % H][:, None]", 0),
    ("dists_not_squared", "ds[row, :m] = d2[a, c]", "ds[row, :m] = np.sqrt(d2[a, c])", 0),
    ("zbuf_from_y", "zb[row, :m] = q[c, 2]", "zb[row, :m] = q[c, 1]", 0),
    ("clouds_not_separated", "lo, hi = int(off[n]), int(off[n + 1])", "lo, hi = 0, int(off[-1])", 0),
    ("bwd_depth_sign", "np.add.at(out[:, 2], q, gz[m, k])", "np.add.at(out[:, 2], q, -gz[m, k])", 0),
    ("bwd_factor_two", "-2.0 * (px[m] - pts[q, 0]) * gd[m, k]", "-1.0 * (px[m] - pts[q, 0]) * gd[m, k]", 0),
    ("bwd_sign", "-2.0 * (py[m] - pts[q, 1]) * gd[m, k]", "2.0 * (py[m] - pts[q, 1]) * gd[m, k]", 0),
    ("bwd_y_uses_px", "-2.0 * (py[m] - pts[q, 1])", "-2.0 * (px[m] - pts[q, 1])", 0),
    ("bwd_padding_counted", "m = idx[:, k] >= 0", "m = idx[:, k] >= -1", 0),
    ("bwd_centre_rows_cols", "py = _centres(H, dt).astype(np.float64)[rem // W]",
     "py = _centres(H, dt).astype(np.float64)[(rem % W) % H]", 0),
]

PIN_NAMES = [n for n, f in inspect.getmembers(T, inspect.isfunction) if n.startswith("test_")]
ARGS = {"test_exact_brute_force": [(s,) for s in range(4)],
        "test_backward_matches_finite_differences": [(0,), (1,)],
        "test_point_band_oracle_equals_whole_oracle": [("points_small",)]}


def _plant(tmp_path, name, orig, new, which):
    src = open(POINTS_SRC).read()
    at = -1
    for _ in range(which + 1):
        at = src.index(orig, at + 1)
    src = src[:at] + new + src[at + len(orig):]
    path = tmp_path / f"points_{name}.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(f"points_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pins_pass(mod, monkeypatch):
    for fn in ("rasterize_points", "rasterize_points_backward"):
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
    import oracle.points as real

    assert _pins_pass(real, monkeypatch)


@pytest.mark.parametrize("name,orig,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, orig, new, which):
    mod = _plant(tmp_path, name, orig, new, which)
    assert not _pins_pass(mod, monkeypatch), f"planted mistake {name} passes every pin"

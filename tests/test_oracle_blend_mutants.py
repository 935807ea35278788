"""The blend oracle's pins are sharp: each plausible mistake planted in a copy
of oracle/blend.py (a dropped or inflated term, a wrong sign, a transposed
quantity), in the forward pass, the backward pass or the per-slot error
scale that sets the GPU tolerance, must make at least one pin of
test_oracle_blend.py fail. The planted copies are imported from a temporary
directory; the real oracle is never modified."""

import importlib.util
import inspect
import os
import sys

import numpy as np
import pytest

import test_oracle_blend as T

BLEND_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "blend.py")

# (name, original text, planted text, which occurrence of the original: 0 = first)
MUTANTS = [
    ("softplus_abs", "return np.maximum(x, 0.0) + np.log1p", "return np.abs(x) + np.log1p", 0),
    ("q_equals_p", "log_q = np.where(filled, -_softplus(-s), 0.0)", "log_q = np.where(filled, -_softplus(s), 0.0)", 0),
    ("zeta_reversed", "zeta = (prm.zfar - z) / (prm.zfar - prm.znear)",
     "zeta = (z - prm.znear) / (prm.zfar - prm.znear)", 0),
    ("background_sign", "log_bg = (prm.eps - zeta_max) / prm.gamma", "log_bg = (prm.eps + zeta_max) / prm.gamma", 0),
    ("denominator_without_background", "den = wn.sum(axis=1) + bgn", "den = wn.sum(axis=1) + 0.0 * bgn", 0),
    ("forward_drops_background", "rgb = np.einsum(\"pk,pkc->pc\", what, c) + bghat[:, None] * bg[None, :]",
     "rgb = np.einsum(\"pk,pkc->pc\", what, c)", 0),
    ("alpha_complement", "alpha = -np.expm1(log_1ma)", "alpha = np.exp(log_1ma)", 0),
    ("bwd_rgb_term_dropped", "g[:, :3], c - rgb[:, None, :]) * what", "g[:, :3], c) * what", 0),
    ("bwd_dist_factor_without_q", "gd = gw * (-q / prm.sigma)", "gd = gw * (-1.0 / prm.sigma)", 0),
    ("bwd_depth_factor", "gz = gw * (-1.0 / ((prm.zfar - prm.znear) * prm.gamma))", "gz = gw * (-1.0 / prm.gamma)", 0),
    ("bwd_alpha_without_coverage_product", "gd = gd + g[:, 3:4] * (-np.exp(log_1ma[:, None] + log_p) / prm.sigma)",
     "gd = gd + g[:, 3:4] * (-np.exp(log_p) / prm.sigma)", 0),
    ("bwd_alpha_sign", "gd = gd + g[:, 3:4] * (-np.exp(", "gd = gd + g[:, 3:4] * (np.exp(", 0),
    ("scale_rgb_term_dropped", "np.abs(c) + np.abs(rgb)[:, None, :]) * what", "np.abs(c)) * what", 0),
    ("scale_weight_dropped", "np.abs(c) + np.abs(rgb)[:, None, :]) * what", "np.abs(c) + np.abs(rgb)[:, None, :])", 0),
    ("scale_alpha_term_dropped",
     "sd = gw * (q / prm.sigma) + g[:, 3:4] * (np.exp(log_1ma[:, None] + log_p) / prm.sigma)",
     "sd = gw * (q / prm.sigma)", 0),
    ("scale_alpha_uses_q", "g[:, 3:4] * (np.exp(log_1ma[:, None] + log_p) / prm.sigma)",
     "g[:, 3:4] * (np.exp(log_1ma[:, None] + log_q) / prm.sigma)", 0),
    ("scale_dist_without_q", "sd = gw * (q / prm.sigma)", "sd = gw * (1.0 / prm.sigma)", 0),
    ("scale_depth_factor", "sz = gw * (1.0 / ((prm.zfar - prm.znear) * prm.gamma))", "sz = gw * (1.0 / prm.gamma)", 0),
    ("scale_inflated", "sz = gw * (1.0 / ((prm.zfar - prm.znear) * prm.gamma))",
     "sz = 4.0 * gw * (1.0 / ((prm.zfar - prm.znear) * prm.gamma))", 0),
    ("linear_domain_weights", "wn = np.exp(log_w - m[:, None])", "wn = np.exp(log_w)", 0),
]

PIN_NAMES = [n for n, f in inspect.getmembers(T, inspect.isfunction) if n.startswith("test_")]
SEEDS = {"test_backward_matches_finite_differences": [4, 5], "test_scale_bounds_every_gradient": [6, 7]}


def _plant(tmp_path, name, orig, new, which):
    src = open(BLEND_SRC).read()
    at = -1
    for _ in range(which + 1):
        at = src.index(orig, at + 1)
    src = src[:at] + new + src[at + len(orig):]
    path = tmp_path / f"blend_{name}.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(f"blend_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod   # the dataclass of the copy looks its module up
    try:
        spec.loader.exec_module(mod)
    finally:
        del sys.modules[spec.name]
    return mod


def _pins_pass(mod, monkeypatch):
    for fn in ("blend_forward", "blend_backward", "blend_backward_scale"):
        monkeypatch.setattr(T, fn, getattr(mod, fn))
    monkeypatch.setattr(T, "BlendParams", mod.BlendParams)
    for name in PIN_NAMES:
        for args in ([(s,) for s in SEEDS[name]] if name in SEEDS else [()]):
            try:
                with np.errstate(all="ignore"):
                    getattr(T, name)(*args)
            except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
                return False
    return True


def test_pins_pass_on_the_real_oracle(monkeypatch):
    import oracle.blend as real

    assert _pins_pass(real, monkeypatch)


@pytest.mark.parametrize("name,orig,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, orig, new, which):
    mod = _plant(tmp_path, name, orig, new, which)
    assert not _pins_pass(mod, monkeypatch), f"planted mistake {name} passes every pin"

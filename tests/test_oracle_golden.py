"""Oracle against the hand-worked cases in tests/golden/hand_cases.json.

Every expected value there was derived on paper from the conventions (see the
file's 'about' and 'citation'), never from either implementation. The
forward checks are exact (binary fractions), in binary32 and binary64.
"""

import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _load():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _val(x, dt):
    if isinstance(x, str):
        assert x.startswith("fl(") and x.endswith(")")
        return dt(np.float32(float(x[3:-1])))
    return dt(x)


def _inputs(case):
    verts = np.asarray(case["verts"], np.float32)
    faces = np.asarray(case["faces"], np.int64)
    offsets = np.asarray(case["offsets"], np.int64)
    return verts, faces, offsets


def _expected(case, dt):
    N = len(case["offsets"]) - 1
    H, W, K = case["H"], case["W"], case["K"]
    p2f = -np.ones((N, H, W, K), np.int64)
    zbuf = -np.ones((N, H, W, K), dt)
    bary = -np.ones((N, H, W, K, 3), dt)
    dists = -np.ones((N, H, W, K), dt)
    for e in case["expect"]:
        n, i, j = e["n"], e["i"], e["j"]
        for k, f in enumerate(e["faces"]):
            p2f[n, i, j, k] = f
            zbuf[n, i, j, k] = _val(e["zbuf"][k], dt)
            bary[n, i, j, k] = [_val(b, dt) for b in e["bary"][k]]
            dists[n, i, j, k] = _val(e["dists"][k], dt)
    return p2f, zbuf, bary, dists


CASES = _load()["cases"]


@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_case_forward(oracle_mod, case, precision):
    dt = np.float32 if precision == "f32" else np.float64
    v, f, o = _inputs(case)
    got = oracle_mod.rasterize(v, f, o, case["H"], case["W"], case["K"], case["blur"], precision=precision)
    exp = _expected(case, dt)
    names = ("pix_to_face", "zbuf", "bary", "dists")
    for name, g, e in zip(names, got, exp):
        if precision == "f64" and name in ("bary",) and case["name"] == "C_blur":
            # fl(0.7)/fl(0.3) are binary32 roundings; binary64 gives 0.7/0.3 to 1e-16
            np.testing.assert_allclose(g, e, rtol=0, atol=1e-7, err_msg=name)
            continue
        np.testing.assert_array_equal(g, e, err_msg=f"{case['name']} {name}")
    # dists = +0.0 (not -0.0) on edge pixels: an edge pixel is not inside
    if case["name"] == "C_blur":
        assert not np.signbit(got[3][0, 0, 3, 0])


@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_hand_case_backward(oracle_mod, precision):
    data = _load()
    cases = {c["name"]: c for c in data["cases"]}
    for bc in data["backward_cases"]:
        case = cases[bc["case"]]
        v, f, o = _inputs(case)
        H, W, K = case["H"], case["W"], case["K"]
        N = len(case["offsets"]) - 1
        p2f = oracle_mod.rasterize(v, f, o, H, W, K, case["blur"], precision=precision)[0]
        px = bc["pixel"]
        for g in bc["grads"]:
            gz = np.zeros((N, H, W, K), np.float32)
            gb = np.zeros((N, H, W, K, 3), np.float32)
            gd = np.zeros((N, H, W, K), np.float32)
            gz[px["n"], px["i"], px["j"], px["slot"]] = g["gz"]
            gb[px["n"], px["i"], px["j"], px["slot"]] = g["gbary"]
            gd[px["n"], px["i"], px["j"], px["slot"]] = g["gd"]
            got = oracle_mod.backward(v, f, o, H, W, K, case["blur"], p2f, gz, gb, gd, precision=precision)
            np.testing.assert_array_equal(got, np.asarray(g["grad_verts"], np.float64),
                                          err_msg=f"{bc['name']} {g}")

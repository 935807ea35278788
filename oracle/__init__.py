"""Python access to the CPU oracle (oracle/raster_oracle.c).

TEST INFRASTRUCTURE ONLY: the plain, slow definition of K-nearest-face mesh
rasterization that the GPU path is checked against. Only tests/,
__graft_entry__.smoke() and the CPU-baseline leg of bench.py may import this
package. It imports nothing from the GPU package, and the GPU package imports
nothing from here.

Parity unpinned: agreement with any existing library's numerics. The pages
print no numeric example, so every pin is a hand-worked case, an exact
rational brute force, an invariant or a finite-difference check.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "raster_oracle.c"), os.path.join(_HERE, "raster_oracle_impl.h")]

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(out_path: str = LIB_PATH, source_dir: str = _HERE, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    src = os.path.join(source_dir, "raster_oracle.c")
    tmp = out_path + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


# Settings bits of the oracle (raster_oracle_impl.h): perspective-correct
# barycentrics, back-face culling, unclipped barycentrics returned.
PERSPECTIVE = 0x2
CULL_BACKFACES = 0x4
UNCLIPPED_BARY = 0x8

_lib = None


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    U32 = ctypes.c_uint32
    for sfx, real in (("f32", ctypes.c_float), ("f64", ctypes.c_double)):
        fn = getattr(lib, f"oracle_raster_{sfx}")
        fn.restype = ctypes.c_int
        fn.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, real, U32, P, I64, P, P, P, P, P]
        fn = getattr(lib, f"oracle_backward_{sfx}")
        fn.restype = ctypes.c_int
        fn.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, real, U32, P, I64, P, P, P, P, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(verts, faces, offsets, precision="f32"):
    vdt = np.float32 if precision == "f32" else np.float64
    verts = np.ascontiguousarray(verts, dtype=vdt).reshape(-1, 3)
    faces = np.ascontiguousarray(faces, dtype=np.int64).reshape(-1, 3)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64).reshape(-1)
    return verts, faces, offsets


def num_threads(lib_path: Optional[str] = None) -> int:
    return int(_load(lib_path).oracle_num_threads())


def rasterize(verts, faces, offsets, H: int, W: int, K: int, blur: float,
              pixels: Optional[np.ndarray] = None, precision: str = "f32",
              with_state: bool = False, lib_path: Optional[str] = None, settings: int = 0):
    """Forward pass on all pixels (pixels=None, outputs [N,H,W,K...]) or on a
    list of flat pixel ids (outputs [len(pixels), K...]).

    Returns (pix_to_face int64, zbuf, bary, dists[, state int32]) as numpy
    arrays of float32 (precision 'f32') or float64 ('f64'). With 'f64' the
    vertices are taken as float64 (float32 inputs widen exactly). `settings`
    is a mask of PERSPECTIVE, CULL_BACKFACES and UNCLIPPED_BARY."""
    lib = _load(lib_path)
    verts, faces, offsets = _prep(verts, faces, offsets, precision)
    N = offsets.shape[0] - 1
    dt = np.float32 if precision == "f32" else np.float64
    if pixels is None:
        shape = (N, H, W, K)
        npix = N * H * W
        pix = None
    else:
        pix = np.ascontiguousarray(pixels, dtype=np.int64).reshape(-1)
        npix = pix.shape[0]
        shape = (npix, K)
    p2f = np.empty(shape, np.int64)
    zbuf = np.empty(shape, dt)
    bary = np.empty(shape + (3,), dt)
    dists = np.empty(shape, dt)
    state = np.empty(shape, np.int32) if with_state else None
    fn = lib.oracle_raster_f32 if precision == "f32" else lib.oracle_raster_f64
    rc = fn(_ptr(verts), verts.shape[0], _ptr(faces), faces.shape[0], _ptr(offsets), N,
            H, W, K, float(blur), int(settings), _ptr(pix), npix,
            _ptr(p2f), _ptr(zbuf), _ptr(bary), _ptr(dists), _ptr(state))
    if rc != 0:
        raise RuntimeError(f"oracle_raster_{precision} failed with code {rc}")
    out = (p2f, zbuf, bary, dists)
    return out + (state,) if with_state else out


def backward(verts, faces, offsets, H: int, W: int, K: int, blur: float, pix_to_face,
             grad_zbuf=None, grad_bary=None, grad_dists=None,
             pixels: Optional[np.ndarray] = None, precision: str = "f32",
             lib_path: Optional[str] = None, settings: int = 0) -> np.ndarray:
    """Backward pass: returns grad_verts [V,3] as float64 (sum of the per-slot
    partials formed in `precision`). Gradient arrays match pix_to_face's
    layout ([N,H,W,K] for all pixels, [len(pixels), K] for a pixel list)."""
    lib = _load(lib_path)
    verts, faces, offsets = _prep(verts, faces, offsets, precision)
    N = offsets.shape[0] - 1
    p2f = np.ascontiguousarray(pix_to_face, dtype=np.int64)
    pix = None if pixels is None else np.ascontiguousarray(pixels, dtype=np.int64).reshape(-1)
    npix = N * H * W if pix is None else pix.shape[0]

    def g(a):
        return None if a is None else np.ascontiguousarray(a, dtype=np.float32)

    gz, gb, gd = g(grad_zbuf), g(grad_bary), g(grad_dists)
    out = np.zeros((verts.shape[0], 3), np.float64)
    fn = lib.oracle_backward_f32 if precision == "f32" else lib.oracle_backward_f64
    rc = fn(_ptr(verts), verts.shape[0], _ptr(faces), faces.shape[0], _ptr(offsets), N,
            H, W, K, float(blur), int(settings), _ptr(pix), npix, _ptr(p2f),
            _ptr(gz), _ptr(gb), _ptr(gd), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_backward_{precision} failed with code {rc}")
    return out

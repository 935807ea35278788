"""MI355X-native K-nearest-face mesh rasterizer (forward and backward).

A thin ctypes binding over libdmr.so, whose C ABI is declared in
include/dmr.h. The functions below only marshal torch tensors (device
memory) and the current HIP stream into that ABI: every step of the
computation runs in the library's HIP kernels. There is no CPU fallback: if
libdmr.so is missing, every call raises.

    rasterize_meshes_fwd / rasterize_meshes_bwd   the two C-ABI entry points
    rasterize_meshes_fwd_ex                       the forward with rasterizer settings
    dmr_blend_fwd / dmr_blend_bwd                 the second stage
    dmr_project_fwd / dmr_project_bwd             the upstream projection
    rasterize_points_fwd / rasterize_points_bwd   point clouds
    rasterize_meshes, project_meshes,
    rasterize_points                              autograd-aware conveniences
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdmr.so")

DMR_MAX_K = 64
DMR_BWD_REUSE_FORWARD_WORKSPACE = 0x1
DMR_RASTER_PERSPECTIVE_CORRECT = 0x2
DMR_RASTER_CULL_BACKFACES = 0x4
DMR_RASTER_UNCLIPPED_BARY = 0x8
STATUS = {0: "DMR_SUCCESS", 1: "DMR_ERROR_INVALID_VALUE", 2: "DMR_ERROR_WORKSPACE_TOO_SMALL",
          3: "DMR_ERROR_HIP", 4: "DMR_ERROR_UNSUPPORTED"}
EXPORTED = [
    "rasterize_meshes_fwd", "rasterize_meshes_fwd_ex", "rasterize_meshes_bwd", "dmr_workspace_min_size", "dmr_workspace_size_hint",
    "dmr_workspace_stats", "dmr_status_string", "dmr_kernel_count",
    "dmr_kernel_name", "dmr_set_kernel_timing", "dmr_set_kernel_timing_mask", "dmr_kernel_timing",
    "dmr_reset_kernel_timing", "dmr_blend_fwd", "dmr_blend_bwd", "dmr_project_fwd", "dmr_project_bwd",
    "rasterize_points_fwd", "rasterize_points_bwd", "dmr_points_workspace_min_size", "dmr_points_workspace_size_hint",
    "rasterize_meshes_fwd_noalloc",
]
DMR_NOALLOC_SCRATCH_BYTES = 128 << 20


class DmrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_string(status)})")


class dmr_blend_params(ctypes.Structure):
    _fields_ = [("sigma", ctypes.c_float), ("gamma", ctypes.c_float), ("znear", ctypes.c_float),
                ("zfar", ctypes.c_float), ("eps", ctypes.c_float), ("background", ctypes.c_float * 3)]


class dmr_stats(ctypes.Structure):
    _fields_ = [("required_bytes", ctypes.c_int64), ("bin_entries", ctypes.c_int64),
                ("bin_capacity", ctypes.c_int64), ("bins", ctypes.c_int64),
                ("overflow_bins", ctypes.c_int64), ("live_faces", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_lib = None


def lib(path: Optional[str] = None):
    """Loads libdmr.so (once) and declares the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m differentiable_mesh_rasterization_amd.build`")
    L = ctypes.CDLL(p)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.rasterize_meshes_fwd.restype = ctypes.c_int
    L.rasterize_meshes_fwd.argtypes = [P, I64, P, I64, P, I64, I32, I32, I32, ctypes.c_float,
                                       P, P, P, P, P, SZ, P]
    L.rasterize_meshes_fwd_ex.restype = ctypes.c_int
    L.rasterize_meshes_fwd_ex.argtypes = [P, I64, P, I64, P, I64, I32, I32, I32, ctypes.c_float,
                                          P, P, P, P, P, SZ, ctypes.c_uint32, P]
    L.rasterize_meshes_fwd_noalloc.restype = ctypes.c_int
    L.rasterize_meshes_fwd_noalloc.argtypes = [P, I64, P, I64, P, I64, I32, I32, I32, ctypes.c_float, P, P, P, P, P]
    L.rasterize_meshes_bwd.restype = ctypes.c_int
    L.rasterize_meshes_bwd.argtypes = [P, I64, P, I64, P, I64, I32, I32, I32, ctypes.c_float, P, P, P, P, P, P, SZ,
                                       ctypes.c_uint32, P]
    L.dmr_workspace_min_size.restype = SZ
    L.dmr_workspace_min_size.argtypes = [I64, I64, I32, I32]
    L.dmr_workspace_size_hint.restype = SZ
    L.dmr_workspace_size_hint.argtypes = [I64, I64, I32, I32, I32, ctypes.c_float]
    L.dmr_workspace_stats.restype = ctypes.c_int
    L.dmr_workspace_stats.argtypes = [P, ctypes.POINTER(dmr_stats), P]
    L.dmr_status_string.restype = ctypes.c_char_p
    L.dmr_status_string.argtypes = [ctypes.c_int]
    L.dmr_kernel_count.restype = I32
    L.dmr_kernel_count.argtypes = []
    L.dmr_kernel_name.restype = ctypes.c_char_p
    L.dmr_kernel_name.argtypes = [I32]
    L.dmr_set_kernel_timing.restype = ctypes.c_int
    L.dmr_set_kernel_timing.argtypes = [I32]
    L.dmr_set_kernel_timing_mask.restype = ctypes.c_int
    L.dmr_set_kernel_timing_mask.argtypes = [ctypes.c_uint32]
    L.dmr_kernel_timing.restype = ctypes.c_int
    L.dmr_kernel_timing.argtypes = [I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.dmr_reset_kernel_timing.restype = ctypes.c_int
    L.dmr_reset_kernel_timing.argtypes = []
    BP = ctypes.POINTER(dmr_blend_params)
    L.dmr_blend_fwd.restype = ctypes.c_int
    L.dmr_blend_fwd.argtypes = [P, P, P, I64, I32, P, I64, BP, P, P]
    L.dmr_blend_bwd.restype = ctypes.c_int
    L.dmr_blend_bwd.argtypes = [P, P, P, I64, I32, P, I64, BP, P, P, P, P]
    L.dmr_project_fwd.restype = ctypes.c_int
    L.dmr_project_fwd.argtypes = [P, I64, P, I64, P, P, P]
    L.dmr_project_bwd.restype = ctypes.c_int
    L.dmr_project_bwd.argtypes = [P, I64, P, I64, P, P, P, P, P]
    L.rasterize_points_fwd.restype = ctypes.c_int
    L.rasterize_points_fwd.argtypes = [P, I64, P, I64, I32, I32, I32, ctypes.c_float, P, P, P, P, SZ, P]
    L.rasterize_points_bwd.restype = ctypes.c_int
    L.rasterize_points_bwd.argtypes = [P, I64, P, I64, I32, I32, I32, P, P, P, P, P]
    L.dmr_points_workspace_min_size.restype = SZ
    L.dmr_points_workspace_min_size.argtypes = [I64, I64, I32, I32]
    L.dmr_points_workspace_size_hint.restype = SZ
    L.dmr_points_workspace_size_hint.argtypes = [I64, I64, I32, I32, I32, ctypes.c_float]
    if path is None:
        _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dmr_status_string(int(status)).decode()


dmr_status_string = status_string


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, device, shape=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ----------------------------------------------------------------------------
# workspace sizes and statistics
# ----------------------------------------------------------------------------

def dmr_workspace_min_size(N: int, F: int, H: int, W: int) -> int:
    return int(lib().dmr_workspace_min_size(N, F, H, W))


def dmr_workspace_size_hint(N: int, F: int, H: int, W: int, K: int, blur_radius: float) -> int:
    return int(lib().dmr_workspace_size_hint(N, F, H, W, K, blur_radius))


def dmr_workspace_stats(workspace: torch.Tensor) -> dict:
    s = dmr_stats()
    rc = lib().dmr_workspace_stats(_ptr(workspace), ctypes.byref(s), _stream_handle(workspace.device))
    if rc != 0:
        raise DmrError("dmr_workspace_stats", rc)
    return {f: getattr(s, f) for f, _ in dmr_stats._fields_ if f != "reserved"}


# ----------------------------------------------------------------------------
# the two entry points
# ----------------------------------------------------------------------------

def rasterize_meshes_fwd(verts: torch.Tensor, faces: torch.Tensor, mesh_face_offsets: torch.Tensor,
                         H: int, W: int, K: int, blur_radius: float,
                         pix_to_face: torch.Tensor, zbuf: torch.Tensor, bary: torch.Tensor,
                         dists: torch.Tensor, workspace: torch.Tensor) -> None:
    """C-ABI forward call on preallocated device tensors (include/dmr.h)."""
    _forward(verts, faces, mesh_face_offsets, H, W, K, blur_radius, pix_to_face, zbuf, bary, dists, workspace,
             None)


def rasterize_meshes_fwd_ex(verts: torch.Tensor, faces: torch.Tensor, mesh_face_offsets: torch.Tensor,
                            H: int, W: int, K: int, blur_radius: float,
                            pix_to_face: torch.Tensor, zbuf: torch.Tensor, bary: torch.Tensor,
                            dists: torch.Tensor, workspace: torch.Tensor, flags: int) -> None:
    """C-ABI forward call with rasterizer settings (a mask of the
    DMR_RASTER_* bits; include/dmr.h)."""
    _forward(verts, faces, mesh_face_offsets, H, W, K, blur_radius, pix_to_face, zbuf, bary, dists, workspace,
             int(flags))


def rasterize_meshes_fwd_noalloc(verts: torch.Tensor, faces: torch.Tensor, mesh_face_offsets: torch.Tensor,
                                 H: int, W: int, K: int, blur_radius: float,
                                 pix_to_face: torch.Tensor, zbuf: torch.Tensor, bary: torch.Tensor,
                                 dists: torch.Tensor) -> None:
    """C-ABI forward call that allocates nothing: the library's per-device
    scratch array stands in for the workspace (include/dmr.h). Calls that
    overlap on one device race."""
    dev = verts.device
    N = mesh_face_offsets.shape[0] - 1
    _check(verts, "verts", torch.float32, dev)
    _check(faces, "faces", torch.int64, dev)
    _check(mesh_face_offsets, "mesh_face_offsets", torch.int64, dev)
    shape = (N, H, W, K)
    _check(pix_to_face, "pix_to_face", torch.int64, dev, shape)
    _check(zbuf, "zbuf", torch.float32, dev, shape)
    _check(bary, "bary", torch.float32, dev, shape + (3,))
    _check(dists, "dists", torch.float32, dev, shape)
    rc = lib().rasterize_meshes_fwd_noalloc(_ptr(verts), verts.shape[0], _ptr(faces), faces.shape[0],
                                            _ptr(mesh_face_offsets), N, H, W, K, float(blur_radius),
                                            _ptr(pix_to_face), _ptr(zbuf), _ptr(bary), _ptr(dists),
                                            _stream_handle(dev))
    if rc != 0:
        raise DmrError("rasterize_meshes_fwd_noalloc", rc)


def _forward(verts, faces, mesh_face_offsets, H, W, K, blur_radius, pix_to_face, zbuf, bary, dists, workspace,
             flags):
    dev = verts.device
    N = mesh_face_offsets.shape[0] - 1
    _check(verts, "verts", torch.float32, dev)
    _check(faces, "faces", torch.int64, dev)
    _check(mesh_face_offsets, "mesh_face_offsets", torch.int64, dev)
    shape = (N, H, W, K)
    _check(pix_to_face, "pix_to_face", torch.int64, dev, shape)
    _check(zbuf, "zbuf", torch.float32, dev, shape)
    _check(bary, "bary", torch.float32, dev, shape + (3,))
    _check(dists, "dists", torch.float32, dev, shape)
    _check(workspace, "workspace", torch.uint8, dev)
    args = (_ptr(verts), verts.shape[0], _ptr(faces), faces.shape[0], _ptr(mesh_face_offsets), N,
            H, W, K, float(blur_radius), _ptr(pix_to_face), _ptr(zbuf), _ptr(bary), _ptr(dists),
            _ptr(workspace), workspace.numel())
    if flags is None:
        rc = lib().rasterize_meshes_fwd(*args, _stream_handle(dev))
        if rc != 0:
            raise DmrError("rasterize_meshes_fwd", rc)
    else:
        rc = lib().rasterize_meshes_fwd_ex(*args, flags, _stream_handle(dev))
        if rc != 0:
            raise DmrError("rasterize_meshes_fwd_ex", rc)


def rasterize_meshes_bwd(verts: torch.Tensor, faces: torch.Tensor, mesh_face_offsets: torch.Tensor,
                         H: int, W: int, K: int, blur_radius: float, pix_to_face: torch.Tensor,
                         grad_zbuf: Optional[torch.Tensor], grad_bary: Optional[torch.Tensor],
                         grad_dists: Optional[torch.Tensor], grad_verts: torch.Tensor,
                         workspace: Optional[torch.Tensor] = None, reuse_forward_workspace: bool = False,
                         settings: int = 0) -> None:
    """C-ABI backward call on preallocated device tensors (include/dmr.h).

    With reuse_forward_workspace=True, `workspace` must be the forward call's
    workspace for these same inputs, unmodified since. `settings` are the
    DMR_RASTER_* bits the forward call was given."""
    dev = verts.device
    N = mesh_face_offsets.shape[0] - 1
    shape = (N, H, W, K)
    _check(verts, "verts", torch.float32, dev)
    _check(faces, "faces", torch.int64, dev)
    _check(mesh_face_offsets, "mesh_face_offsets", torch.int64, dev)
    _check(pix_to_face, "pix_to_face", torch.int64, dev, shape)
    _check(grad_zbuf, "grad_zbuf", torch.float32, dev, shape, optional=True)
    _check(grad_bary, "grad_bary", torch.float32, dev, shape + (3,), optional=True)
    _check(grad_dists, "grad_dists", torch.float32, dev, shape, optional=True)
    _check(grad_verts, "grad_verts", torch.float32, dev, tuple(verts.shape))
    _check(workspace, "workspace", torch.uint8, dev, optional=not reuse_forward_workspace)
    flags = (DMR_BWD_REUSE_FORWARD_WORKSPACE if reuse_forward_workspace else 0) | int(settings)
    rc = lib().rasterize_meshes_bwd(
        _ptr(verts), verts.shape[0], _ptr(faces), faces.shape[0], _ptr(mesh_face_offsets), N,
        H, W, K, float(blur_radius), _ptr(pix_to_face), _ptr(grad_zbuf), _ptr(grad_bary), _ptr(grad_dists),
        _ptr(grad_verts), _ptr(workspace), 0 if workspace is None else workspace.numel(), flags,
        _stream_handle(dev))
    if rc != 0:
        raise DmrError("rasterize_meshes_bwd", rc)


def blend_params(sigma: float = 1e-4, gamma: float = 1e-4, znear: float = 1.0, zfar: float = 100.0,
                 eps: float = 1e-10, background=(1.0, 1.0, 1.0)) -> dmr_blend_params:
    return dmr_blend_params(sigma, gamma, znear, zfar, eps, (ctypes.c_float * 3)(*background))


def _blend_inputs(pix_to_face, zbuf, dists, face_colors):
    dev = pix_to_face.device
    K = pix_to_face.shape[-1]
    _check(pix_to_face, "pix_to_face", torch.int64, dev)
    _check(zbuf, "zbuf", torch.float32, dev, tuple(pix_to_face.shape))
    _check(dists, "dists", torch.float32, dev, tuple(pix_to_face.shape))
    _check(face_colors, "face_colors", torch.float32, dev)
    if face_colors.dim() != 2 or face_colors.shape[1] != 3:
        raise ValueError("face_colors must be [F, 3]")
    return dev, pix_to_face.numel() // K, K


def dmr_blend_fwd(pix_to_face: torch.Tensor, zbuf: torch.Tensor, dists: torch.Tensor, face_colors: torch.Tensor,
                  params: dmr_blend_params, rgba: torch.Tensor) -> None:
    """C-ABI second-stage blend on preallocated device tensors (include/dmr.h):
    rgba [..., 4] from the forward pass's [..., K] outputs."""
    dev, P, K = _blend_inputs(pix_to_face, zbuf, dists, face_colors)
    _check(rgba, "rgba", torch.float32, dev, tuple(pix_to_face.shape[:-1]) + (4,))
    rc = lib().dmr_blend_fwd(_ptr(pix_to_face), _ptr(zbuf), _ptr(dists), P, K, _ptr(face_colors),
                             face_colors.shape[0], ctypes.byref(params), _ptr(rgba), _stream_handle(dev))
    if rc != 0:
        raise DmrError("dmr_blend_fwd", rc)


def dmr_blend_bwd(pix_to_face: torch.Tensor, zbuf: torch.Tensor, dists: torch.Tensor, face_colors: torch.Tensor,
                  params: dmr_blend_params, grad_rgba: torch.Tensor, grad_zbuf: torch.Tensor,
                  grad_dists: torch.Tensor) -> None:
    """C-ABI backward of the blend: grad_zbuf, grad_dists [..., K] from grad_rgba [..., 4]."""
    dev, P, K = _blend_inputs(pix_to_face, zbuf, dists, face_colors)
    _check(grad_rgba, "grad_rgba", torch.float32, dev, tuple(pix_to_face.shape[:-1]) + (4,))
    _check(grad_zbuf, "grad_zbuf", torch.float32, dev, tuple(pix_to_face.shape))
    _check(grad_dists, "grad_dists", torch.float32, dev, tuple(pix_to_face.shape))
    rc = lib().dmr_blend_bwd(_ptr(pix_to_face), _ptr(zbuf), _ptr(dists), P, K, _ptr(face_colors),
                             face_colors.shape[0], ctypes.byref(params), _ptr(grad_rgba), _ptr(grad_zbuf),
                             _ptr(grad_dists), _stream_handle(dev))
    if rc != 0:
        raise DmrError("dmr_blend_bwd", rc)


def _project_inputs(verts_world, mesh_vert_offsets, cameras):
    dev = verts_world.device
    _check(verts_world, "verts_world", torch.float32, dev)
    if verts_world.dim() != 2 or verts_world.shape[1] != 3:
        raise ValueError("verts_world must be [V, 3]")
    _check(mesh_vert_offsets, "mesh_vert_offsets", torch.int64, dev)
    N = mesh_vert_offsets.shape[0] - 1
    _check(cameras, "cameras", torch.float32, dev, (N, 4, 4))
    return dev, verts_world.shape[0], N


def dmr_project_fwd(verts_world: torch.Tensor, mesh_vert_offsets: torch.Tensor, cameras: torch.Tensor,
                    verts_ndc: torch.Tensor) -> None:
    """C-ABI projection on preallocated device tensors (include/dmr.h)."""
    dev, V, N = _project_inputs(verts_world, mesh_vert_offsets, cameras)
    _check(verts_ndc, "verts_ndc", torch.float32, dev, (V, 3))
    rc = lib().dmr_project_fwd(_ptr(verts_world), V, _ptr(mesh_vert_offsets), N, _ptr(cameras), _ptr(verts_ndc),
                               _stream_handle(dev))
    if rc != 0:
        raise DmrError("dmr_project_fwd", rc)


def dmr_project_bwd(verts_world: torch.Tensor, mesh_vert_offsets: torch.Tensor, cameras: torch.Tensor,
                    grad_verts_ndc: torch.Tensor, grad_verts_world: torch.Tensor,
                    grad_cameras: Optional[torch.Tensor] = None) -> None:
    """C-ABI backward of the projection (grad_cameras optional)."""
    dev, V, N = _project_inputs(verts_world, mesh_vert_offsets, cameras)
    _check(grad_verts_ndc, "grad_verts_ndc", torch.float32, dev, (V, 3))
    _check(grad_verts_world, "grad_verts_world", torch.float32, dev, (V, 3))
    _check(grad_cameras, "grad_cameras", torch.float32, dev, (N, 4, 4), optional=True)
    rc = lib().dmr_project_bwd(_ptr(verts_world), V, _ptr(mesh_vert_offsets), N, _ptr(cameras),
                               _ptr(grad_verts_ndc), _ptr(grad_verts_world), _ptr(grad_cameras),
                               _stream_handle(dev))
    if rc != 0:
        raise DmrError("dmr_project_bwd", rc)


def dmr_points_workspace_min_size(N: int, P: int, H: int, W: int) -> int:
    return int(lib().dmr_points_workspace_min_size(N, P, H, W))


def dmr_points_workspace_size_hint(N: int, P: int, H: int, W: int, K: int, radius: float) -> int:
    return int(lib().dmr_points_workspace_size_hint(N, P, H, W, K, radius))


def rasterize_points_fwd(points: torch.Tensor, cloud_offsets: torch.Tensor, H: int, W: int, K: int, radius: float,
                         idx: torch.Tensor, zbuf: torch.Tensor, dists: torch.Tensor, workspace: torch.Tensor) -> None:
    """C-ABI point rasterization on preallocated device tensors (include/dmr.h)."""
    dev = points.device
    N = cloud_offsets.shape[0] - 1
    _check(points, "points", torch.float32, dev)
    _check(cloud_offsets, "cloud_offsets", torch.int64, dev)
    shape = (N, H, W, K)
    _check(idx, "idx", torch.int64, dev, shape)
    _check(zbuf, "zbuf", torch.float32, dev, shape)
    _check(dists, "dists", torch.float32, dev, shape)
    _check(workspace, "workspace", torch.uint8, dev)
    rc = lib().rasterize_points_fwd(_ptr(points), points.shape[0], _ptr(cloud_offsets), N, H, W, K, float(radius),
                                    _ptr(idx), _ptr(zbuf), _ptr(dists), _ptr(workspace), workspace.numel(),
                                    _stream_handle(dev))
    if rc != 0:
        raise DmrError("rasterize_points_fwd", rc)


def rasterize_points_bwd(points: torch.Tensor, cloud_offsets: torch.Tensor, H: int, W: int, K: int,
                         idx: torch.Tensor, grad_zbuf: Optional[torch.Tensor], grad_dists: Optional[torch.Tensor],
                         grad_points: torch.Tensor) -> None:
    """C-ABI backward of the point rasterization (include/dmr.h)."""
    dev = points.device
    N = cloud_offsets.shape[0] - 1
    shape = (N, H, W, K)
    _check(points, "points", torch.float32, dev)
    _check(cloud_offsets, "cloud_offsets", torch.int64, dev)
    _check(idx, "idx", torch.int64, dev, shape)
    _check(grad_zbuf, "grad_zbuf", torch.float32, dev, shape, optional=True)
    _check(grad_dists, "grad_dists", torch.float32, dev, shape, optional=True)
    _check(grad_points, "grad_points", torch.float32, dev, tuple(points.shape))
    rc = lib().rasterize_points_bwd(_ptr(points), points.shape[0], _ptr(cloud_offsets), N, H, W, K, _ptr(idx),
                                    _ptr(grad_zbuf), _ptr(grad_dists), _ptr(grad_points), _stream_handle(dev))
    if rc != 0:
        raise DmrError("rasterize_points_bwd", rc)


# ----------------------------------------------------------------------------
# convenience: allocation + autograd
# ----------------------------------------------------------------------------

class Workspace:
    """Grow-only forward workspace for one device. The first call on a shape
    uses the library's size hint; calls made with too small a workspace stay
    exact (overflowing bins take the slow path), and `grow()` reads the size
    the last call needed."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = torch.empty(0, dtype=torch.uint8, device=self.device)

    def ensure(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        return self.buf

    def grow(self) -> dict:
        stats = dmr_workspace_stats(self.buf)
        self.ensure(stats["required_bytes"])
        return stats


_workspaces = {}


def workspace_for(device) -> Workspace:
    device = torch.device(device)
    if device not in _workspaces:
        _workspaces[device] = Workspace(device)
    return _workspaces[device]


def _alloc_outputs(N, H, W, K, device):
    return (torch.empty((N, H, W, K), dtype=torch.int64, device=device),
            torch.empty((N, H, W, K), dtype=torch.float32, device=device),
            torch.empty((N, H, W, K, 3), dtype=torch.float32, device=device),
            torch.empty((N, H, W, K), dtype=torch.float32, device=device))


class _RasterizeMeshes(torch.autograd.Function):
    @staticmethod
    def forward(ctx, verts, faces, offsets, H, W, K, blur_radius, settings):
        N = offsets.shape[0] - 1
        out = _alloc_outputs(N, H, W, K, verts.device)
        # Each call owns its workspace: the backward pass reuses its face
        # records and bin lists, so it must survive until then.
        ws = torch.empty(dmr_workspace_size_hint(N, faces.shape[0], H, W, K, blur_radius), dtype=torch.uint8,
                         device=verts.device)
        rasterize_meshes_fwd_ex(verts, faces, offsets, H, W, K, blur_radius, *out, ws, settings)
        ctx.save_for_backward(verts, faces, offsets, out[0], ws)
        ctx.dims = (H, W, K, blur_radius, settings)
        ctx.mark_non_differentiable(out[0])
        return out

    @staticmethod
    def backward(ctx, g_p2f, g_zbuf, g_bary, g_dists):
        verts, faces, offsets, p2f, ws = ctx.saved_tensors
        H, W, K, blur_radius, settings = ctx.dims
        grad_verts = torch.empty_like(verts)

        def c(g):
            return None if g is None else g.contiguous()

        rasterize_meshes_bwd(verts, faces, offsets, H, W, K, blur_radius, p2f, c(g_zbuf), c(g_bary), c(g_dists),
                             grad_verts, ws, reuse_forward_workspace=True, settings=settings)
        return grad_verts, None, None, None, None, None, None, None


def rasterize_meshes(verts: torch.Tensor, faces: torch.Tensor, mesh_face_offsets: torch.Tensor,
                     image_size: Tuple[int, int], faces_per_pixel: int = 1, blur_radius: float = 0.0,
                     perspective_correct: bool = False, cull_backfaces: bool = False,
                     clip_barycentric_coords: bool = True):
    """Rasterizes a packed batch of meshes on the GPU.

    verts [V,3] float32 (x, y NDC, z depth), faces [F,3] int64, mesh_face_offsets
    [N+1] int64. Returns (pix_to_face, zbuf, bary, dists); zbuf, bary and dists
    are differentiable with respect to verts. The three settings map to the
    DMR_RASTER_* bits of include/dmr.h."""
    H, W = image_size
    settings = ((DMR_RASTER_PERSPECTIVE_CORRECT if perspective_correct else 0)
                | (DMR_RASTER_CULL_BACKFACES if cull_backfaces else 0)
                | (0 if clip_barycentric_coords else DMR_RASTER_UNCLIPPED_BARY))
    return _RasterizeMeshes.apply(verts, faces, mesh_face_offsets, int(H), int(W), int(faces_per_pixel),
                                  float(blur_radius), settings)


class _ProjectMeshes(torch.autograd.Function):
    @staticmethod
    def forward(ctx, verts_world, mesh_vert_offsets, cameras):
        out = torch.empty_like(verts_world)
        dmr_project_fwd(verts_world, mesh_vert_offsets, cameras, out)
        ctx.save_for_backward(verts_world, mesh_vert_offsets, cameras)
        return out

    @staticmethod
    def backward(ctx, g):
        verts_world, offs, cameras = ctx.saved_tensors
        gv = torch.empty_like(verts_world)
        gc = torch.empty_like(cameras) if ctx.needs_input_grad[2] else None
        dmr_project_bwd(verts_world, offs, cameras, g.contiguous(), gv, gc)
        return gv, None, gc


def project_meshes(verts_world: torch.Tensor, mesh_vert_offsets: torch.Tensor, cameras: torch.Tensor):
    """Projects a packed batch of meshes (one 4x4 camera per mesh) to the
    rasterizer's screen space; differentiable with respect to verts_world
    and cameras."""
    return _ProjectMeshes.apply(verts_world, mesh_vert_offsets, cameras)


class _RasterizePoints(torch.autograd.Function):
    @staticmethod
    def forward(ctx, points, offsets, H, W, K, radius):
        N = offsets.shape[0] - 1
        dev = points.device
        idx = torch.empty((N, H, W, K), dtype=torch.int64, device=dev)
        zbuf = torch.empty((N, H, W, K), dtype=torch.float32, device=dev)
        dists = torch.empty((N, H, W, K), dtype=torch.float32, device=dev)
        ws = torch.empty(dmr_points_workspace_size_hint(N, points.shape[0], H, W, K, radius), dtype=torch.uint8,
                         device=dev)
        rasterize_points_fwd(points, offsets, H, W, K, radius, idx, zbuf, dists, ws)
        ctx.save_for_backward(points, offsets, idx)
        ctx.dims = (H, W, K)
        ctx.mark_non_differentiable(idx)
        return idx, zbuf, dists

    @staticmethod
    def backward(ctx, g_idx, g_zbuf, g_dists):
        points, offsets, idx = ctx.saved_tensors
        H, W, K = ctx.dims
        grad = torch.empty_like(points)

        def c(g):
            return None if g is None else g.contiguous()

        rasterize_points_bwd(points, offsets, H, W, K, idx, c(g_zbuf), c(g_dists), grad)
        return grad, None, None, None, None, None


def rasterize_points(points: torch.Tensor, cloud_offsets: torch.Tensor, image_size: Tuple[int, int],
                     points_per_pixel: int = 1, radius: float = 0.01):
    """Rasterizes a packed batch of point clouds on the GPU: (idx, zbuf,
    dists), zbuf and dists differentiable with respect to points."""
    H, W = image_size
    return _RasterizePoints.apply(points, cloud_offsets, int(H), int(W), int(points_per_pixel), float(radius))


# ----------------------------------------------------------------------------
# per-kernel timing (measurement only)
# ----------------------------------------------------------------------------

def kernel_names():
    L = lib()
    return [L.dmr_kernel_name(i).decode() for i in range(L.dmr_kernel_count())]


def set_kernel_timing(enable: bool) -> None:
    rc = lib().dmr_set_kernel_timing(1 if enable else 0)
    if rc != 0:
        raise DmrError("dmr_set_kernel_timing", rc)


def set_kernel_timing_only(names) -> None:
    """Times only the named kernels (see kernel_names())."""
    ids = kernel_names()
    mask = 0
    for n in names:
        mask |= 1 << ids.index(n)
    rc = lib().dmr_set_kernel_timing_mask(mask)
    if rc != 0:
        raise DmrError("dmr_set_kernel_timing_mask", rc)


def reset_kernel_timing() -> None:
    rc = lib().dmr_reset_kernel_timing()
    if rc != 0:
        raise DmrError("dmr_reset_kernel_timing", rc)


def kernel_timing() -> dict:
    """{kernel name: (total ms, launches)} since the last reset."""
    L = lib()
    out = {}
    for i, name in enumerate(kernel_names()):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        rc = L.dmr_kernel_timing(i, ctypes.byref(ms), ctypes.byref(n))
        if rc != 0:
            raise DmrError("dmr_kernel_timing", rc)
        out[name] = (ms.value, n.value)
    return out

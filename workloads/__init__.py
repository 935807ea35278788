"""Seeded synthetic inputs for the mesh rasterizer.

This package only draws geometry, per-face colours, cameras, point clouds and upstream gradients. It holds none of the
rasterizer's arithmetic, so both the CPU oracle (through the tests) and the
GPU path (through the tests and the benchmark) can consume the same arrays
without sharing any code of the method itself.
"""

from .meshes import (  # noqa: F401
    CONFIGS,
    Workload,
    icosphere,
    make_workload,
    upstream_grads,
    sample_pixels,
    masked_upstream_grads,
    face_colors,
    blend_upstream_grads,
    vert_offsets,
    projection_inputs,
    projection_upstream_grads,
    PointWorkload,
    POINT_CONFIGS,
    make_point_workload,
    point_upstream_grads,
)

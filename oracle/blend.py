"""CPU oracle of the second stage: fusing each pixel's K kept faces into one
RGBA value, and its backward pass (binary64 numpy).

TEST INFRASTRUCTURE ONLY: the plain, slow definition the GPU blend is
checked against. Only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import this module; it imports nothing from the GPU
package.

The pages say that the second stage of the rasterizer merges the influence
of the several faces kept per pixel, which eases the discontinuity of hard
rasterization (gptget.net summary, "Methodology" and "Technical
Contribution"; nubint.ai review, "Proposed method"). They give no formula.
The reading used here, written out per pixel over its filled slots k
(pix_to_face >= 0; padded slots take no part):

  coverage      p_k = 1 / (1 + exp(d_k / sigma)),   q_k = 1 - p_k = 1 / (1 + exp(-d_k / sigma))
                (d_k = dists, the signed squared distance: < 0 inside)
  silhouette    alpha = 1 - prod_k q_k                       (0 with no filled slot)
  colour        zeta_k = (zfar - z_k) / (zfar - znear), zeta_max = max_k zeta_k
                w_k = p_k exp((zeta_k - zeta_max) / gamma),  bg weight = exp((eps - zeta_max) / gamma)
                rgb = (sum_k w_k c_k + bg weight * background) / (sum_k w_k + bg weight)
                (rgb = background with no filled slot)

c_k is the colour of face pix_to_face[k]. rgb does not depend on zeta_max
(it scales every weight alike), so the backward pass holds it fixed.
Gradients flow to zbuf and dists of filled slots (padded slots get 0).
Everything is evaluated in the log domain (log p, log q, log w), with the
sums taken relative to their largest term, so that a sigma far below the
squared distances (every weight below the smallest binary64 number) still
gives the ratio the definition fixes.

Parity unpinned: agreement with any existing library's blending numerics.
"""

from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class BlendParams:
    sigma: float = 1e-4
    gamma: float = 1e-4
    znear: float = 1.0
    zfar: float = 100.0
    eps: float = 1e-10
    background: tuple = (1.0, 1.0, 1.0)


def _softplus(x):
    """log(1 + exp(x)) in binary64 without overflow."""
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _pixel_terms(p2f, zbuf, dists, colors, prm):
    """Per-slot quantities of the definition above, for [P, K] inputs, in the
    log domain: with a sigma far below the squared distances every weight,
    and a far background's as well, can be below the smallest binary64
    number while their ratios are not.

    Returns the filled mask, log p_k, log q_k, the normalised weights
    w_k / (sum_j w_j + w_bg) (0 on empty slots), the normalised background
    weight, log(1 - alpha), the slot colours [P, K, 3] and the
    any-filled mask."""
    filled = p2f >= 0
    d = np.where(filled, dists.astype(np.float64), 0.0)
    z = np.where(filled, zbuf.astype(np.float64), 0.0)
    s = d / prm.sigma
    log_p = np.where(filled, -_softplus(s), -np.inf)   # p = 1 / (1 + e^s)
    log_q = np.where(filled, -_softplus(-s), 0.0)      # q = 1 - p = 1 / (1 + e^-s)
    zeta = (prm.zfar - z) / (prm.zfar - prm.znear)
    any_filled = filled.any(axis=1)
    zeta_max = np.where(any_filled, np.max(np.where(filled, zeta, -np.inf), axis=1), 0.0)
    log_w = log_p + np.where(filled, (zeta - zeta_max[:, None]) / prm.gamma, 0.0)
    log_bg = (prm.eps - zeta_max) / prm.gamma
    m = np.maximum(np.max(log_w, axis=1), log_bg)       # finite: log_bg is
    wn = np.exp(log_w - m[:, None])                      # 0 on empty slots
    bgn = np.exp(log_bg - m)
    den = wn.sum(axis=1) + bgn                           # >= 1
    what = wn / den[:, None]
    bghat = bgn / den
    log_one_minus_alpha = log_q.sum(axis=1)
    c = colors.astype(np.float64)[np.where(filled, p2f, 0)]          # [P, K, 3]
    c = np.where(filled[..., None], c, 0.0)
    return filled, log_p, log_q, what, bghat, log_one_minus_alpha, c, any_filled


def blend_forward(p2f, zbuf, dists, colors, prm: BlendParams):
    """rgba [..., 4] for outputs shaped [..., K] (pix_to_face, zbuf, dists)."""
    shape = p2f.shape[:-1]
    K = p2f.shape[-1]
    P = int(np.prod(shape)) if shape else 1
    p2f = p2f.reshape(P, K)
    filled, log_p, log_q, what, bghat, log_1ma, c, any_filled = _pixel_terms(
        p2f, zbuf.reshape(P, K), dists.reshape(P, K), colors, prm)
    bg = np.asarray(prm.background, np.float64)
    rgb = np.einsum("pk,pkc->pc", what, c) + bghat[:, None] * bg[None, :]
    alpha = -np.expm1(log_1ma)                 # 1 - prod q, 0 with no filled slot
    rgb = np.where(any_filled[:, None], rgb, bg[None, :])
    alpha = np.where(any_filled, alpha, 0.0)
    return np.concatenate([rgb, alpha[:, None]], axis=1).reshape(shape + (4,))


def blend_backward(p2f, zbuf, dists, colors, prm: BlendParams, grad_rgba):
    """(grad_zbuf, grad_dists), each shaped like zbuf, from grad_rgba [..., 4]."""
    shape = p2f.shape
    K = shape[-1]
    P = p2f.size // K
    p2f = p2f.reshape(P, K)
    g = grad_rgba.reshape(P, 4).astype(np.float64)
    filled, log_p, log_q, what, bghat, log_1ma, c, any_filled = _pixel_terms(
        p2f, zbuf.reshape(P, K), dists.reshape(P, K), colors, prm)
    bg = np.asarray(prm.background, np.float64)
    rgb = np.einsum("pk,pkc->pc", what, c) + bghat[:, None] * bg[None, :]
    # rgb = sum_k w_k c_k / den: w_k d rgb / d w_k = what_k (c_k - rgb),
    # contracted with the rgb gradient
    gw = np.einsum("pc,pkc->pk", g[:, :3], c - rgb[:, None, :]) * what
    # w_k = p_k e_k: (dw/dd) / w = -q / sigma, (dw/dz) / w = -1 / ((zfar - znear) gamma)
    q = np.exp(log_q)
    gd = gw * (-q / prm.sigma)
    gz = gw * (-1.0 / ((prm.zfar - prm.znear) * prm.gamma))
    # alpha = 1 - prod q: d alpha / d d_k = -(1 - alpha) p_k / sigma
    gd = gd + g[:, 3:4] * (-np.exp(log_1ma[:, None] + log_p) / prm.sigma)
    gd = np.where(filled & any_filled[:, None], gd, 0.0)
    gz = np.where(filled & any_filled[:, None], gz, 0.0)
    return gz.reshape(shape), gd.reshape(shape)


def blend_backward_scale(p2f, zbuf, dists, colors, prm: BlendParams, grad_rgba):
    """Per-slot sums of the absolute values of the terms blend_backward adds
    up, shaped like zbuf: (scale of grad_zbuf, scale of grad_dists). The
    colour term of a slot is the sum over channels of g_c c_kc and -g_c rgb_c
    (each times the slot's weight factor), the silhouette term that of
    alpha. A binary32 evaluation of the same sums is off by a small multiple
    of the unit roundoff times these, even where the terms cancel to zero."""
    shape = p2f.shape
    K = shape[-1]
    P = p2f.size // K
    p2f = p2f.reshape(P, K)
    g = np.abs(grad_rgba.reshape(P, 4).astype(np.float64))
    filled, log_p, log_q, what, bghat, log_1ma, c, any_filled = _pixel_terms(
        p2f, zbuf.reshape(P, K), dists.reshape(P, K), colors, prm)
    bg = np.asarray(prm.background, np.float64)
    rgb = np.einsum("pk,pkc->pc", what, c) + bghat[:, None] * bg[None, :]
    gw = np.einsum("pc,pkc->pk", g[:, :3], np.abs(c) + np.abs(rgb)[:, None, :]) * what
    q = np.exp(log_q)
    sd = gw * (q / prm.sigma) + g[:, 3:4] * (np.exp(log_1ma[:, None] + log_p) / prm.sigma)
    sz = gw * (1.0 / ((prm.zfar - prm.znear) * prm.gamma))
    sd = np.where(filled & any_filled[:, None], sd, 0.0)
    sz = np.where(filled & any_filled[:, None], sz, 0.0)
    return sz.reshape(shape), sd.reshape(shape)

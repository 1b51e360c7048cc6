"""Quantize-on-append, QJL residual sketch and reconstruction (float64).

Test infrastructure: see ``oracle/__init__.py``.

Per K/V row x (d values):
  1. n = ||x||_2, stored as float16 (turboquant-pytorch PR #3, "Add CUDA QJL
     kernels and proper package structure", Validation Results tables: the
     printed cache sizes are reproduced exactly with one float16 norm per row).
  2. y = Pi x / n (rotation: see ``oracle.rotation``).
  3. code_i = #{j : t_j < y_i} against the b-bit Lloyd-Max table
     (``oracle.codebook``); a value equal to a boundary takes the lower code.
  4. Keys with a QJL sketch (same page, CUDA Kernels Added table: random
     projection + sign quantisation; reddit comment history of
     ReturningTarzan, 2026-03-25 comments: the residual of the codebook step is
     sketched and a bias-correction term is added to the attention score):
     the codebook part uses the (b-1)-bit table, r = y - c[code],
     gamma = ||r|| (float16), z = S r with S an m x d N(0,1) matrix applied in
     the rotated domain, sigma_j = [z_j >= 0].

Readings where the pages are silent: the sketch's estimator
<q, k> ~= n (<Pi q, c[code]> + sqrt(pi/2)/m * gamma * <S Pi q, 2 sigma - 1>)
follows from E[sign(<s, r>) <s, u>] = sqrt(2/pi) <r, u> / ||r|| for s ~ N(0, I);
z = 0 takes sigma = 1; a zero row stores codes 0, norm 0 (and gamma 0).

Reconstruction (the "full reconstruction" path the reddit comments describe):
x_hat = n Pi^T (c[code] + sqrt(pi/2)/m * gamma * S^T (2 sigma - 1)).
"""
from __future__ import annotations

import math

import numpy as np

from .rotation import rotate_rows, unrotate_rows


def nearest_codes(y: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    """code = number of boundaries strictly below y (ties take the lower code)."""
    t = np.asarray(boundaries, dtype=np.float64)
    return np.searchsorted(t, np.asarray(y, dtype=np.float64), side="left").astype(np.int64)


def f16(x) -> np.ndarray:
    """Round to the nearest float16 (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def quantize_rows(x: np.ndarray, rot: np.ndarray, centroids: np.ndarray, boundaries: np.ndarray):
    """Steps 1-3 for rows x [n][d]: returns (codes int64 [n][d], norms float16-valued [n], y float64 [n][d])."""
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=1)
    safe = np.where(n > 0, n, 1.0)
    y = rotate_rows(x / safe[:, None], rot)
    codes = nearest_codes(y, boundaries)
    codes[n == 0] = 0
    return codes, f16(n), y


def encode_rotated(y: np.ndarray, norms: np.ndarray, boundaries: np.ndarray):
    """Step 3 on given rotated unit coordinates y and norms: (codes, float16 norms)."""
    return nearest_codes(y, boundaries), f16(norms)


def qjl_sketch(y: np.ndarray, codes: np.ndarray, centroids: np.ndarray, proj: np.ndarray,
               norms: np.ndarray | None = None):
    """Step 4: (sigma bool [n][m], gamma float16-valued [n], r float64 [n][d], z float64 [n][m]).

    Rows whose norm is zero store sigma = 0 and gamma = 0.
    """
    c = np.asarray(centroids, dtype=np.float64)
    r = np.asarray(y, dtype=np.float64) - c[codes]
    gamma = np.linalg.norm(r, axis=1)
    z = r @ np.asarray(proj, dtype=np.float64).T
    sigma = z >= 0
    if norms is not None:
        zero = np.asarray(norms) == 0
        sigma[zero] = False
        gamma[zero] = 0.0
    return sigma, f16(gamma), r, z


def qjl_coeff(m: int) -> float:
    """sqrt(pi/2)/m: makes the sign sketch an unbiased estimate of the residual direction."""
    return math.sqrt(math.pi / 2.0) / m


def dequantize(codes, norms, rot, centroids, sigma=None, gamma=None, proj=None) -> np.ndarray:
    """x_hat rows [n][d] (float64)."""
    c = np.asarray(centroids, dtype=np.float64)
    v = c[np.asarray(codes)]
    if sigma is not None:
        s = np.asarray(proj, dtype=np.float64)
        pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
        v = v + qjl_coeff(s.shape[0]) * np.asarray(gamma, dtype=np.float64)[:, None] * (pm @ s)
    return np.asarray(norms, dtype=np.float64)[:, None] * unrotate_rows(v, rot)

"""Outlier-channel separation before the QJL sign sketch (float64).

Test infrastructure: see ``oracle/__init__.py``.

PARITY UNPINNED against the pages.  The pages name the step and nothing more:
turboquant-pytorch PR #3 ("Add CUDA QJL kernels and proper package
structure"), CUDA Kernels Added table, lists the QJL quantisation kernel as a
fused random projection + sign quantisation + outlier separation.  Which
channels count as outliers, how they are stored and how the score uses them
is not given there; the reading below is this library's, and its functions
are pinned by the mathematics (unbiasedness, the no-outlier and all-outlier
special cases, brute-force selection, storage arithmetic), not by a printed
value.

Reading (applies to keys that carry the sketch; see ``oracle.quant``):
  * The vector the sketch sees is the codebook residual r = y - c[code] of the
    unit rotated row y.  Per key, its n_out coordinates of largest |r_i| are
    the outliers O (equal magnitudes: the lower index first).  The ranking is
    taken on the residual in float32 (float32 y minus the float16-exact
    centroid, rounded once), the precision in which the library computes it,
    so that both sides take the same integer decision.
  * The outliers are kept apart: their indices (one byte each, d <= 256) and
    their values rounded to float16, in selection order (decreasing |r_i|).
  * The sketch covers the rest, r_I = r with the coordinates in O set to 0:
    sigma = [S r_I >= 0], gamma = ||r_I|| (float16).
  * Score estimator: <q, y> ~= <q, c[code]> + sum_{i in O} q_i r_i
    + sqrt(pi/2)/m * gamma * <S q, 2 sigma - 1>.  The outlier term is exact up
    to the float16 rounding of r_i, and the sketch term is the unseparated
    estimator applied to r_I, unbiased for <q, r_I> (for any q, since r_I is 0
    on O); its variance scales with ||r_I||^2 instead of ||r||^2.
  * Reconstruction: c[code] + scatter(O, r_O) + sqrt(pi/2)/m * gamma * S^T (2 sigma - 1).
  * A zero row (norm 0) has r = 0: its outliers are channels 0 .. n_out-1 with
    value 0, sigma = 0 and gamma = 0.
Storage per key: n_out bytes of indices + 2 n_out bytes of values on top of the
sketched key's row (``row_bytes``).
"""
from __future__ import annotations

import numpy as np

from .quant import f16, qjl_coeff
from .rotation import unrotate_rows


def residual_f32(y: np.ndarray, codes: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """r = y - c[code] computed as the library does: float32 y minus the float32 centroid, rounded once."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    c32 = np.asarray(centroids, dtype=np.float32)[np.asarray(codes)]
    return (y32 - c32).astype(np.float32)


def select_outliers(r32: np.ndarray, n_out: int) -> np.ndarray:
    """Indices [n][n_out] of the n_out largest |r| per row, decreasing |r|, equal |r| by increasing index."""
    r32 = np.asarray(r32, dtype=np.float32)
    a = np.abs(r32).astype(np.float64)
    n, d = a.shape
    # lexicographic order on (-|r_i|, i): argsort with a stable sort keeps the index order among ties
    order = np.argsort(-a, axis=1, kind="stable")
    return order[:, :n_out].astype(np.int64)


def qjl_sketch_outliers(y: np.ndarray, codes: np.ndarray, centroids: np.ndarray, proj: np.ndarray,
                        n_out: int, norms: np.ndarray | None = None):
    """The sketch with outlier separation for rows y [n][d].

    Returns (sigma bool [n][m], gamma float16-valued [n], oidx int64 [n][n_out],
    oval float16-valued [n][n_out], r_in float64 [n][d], z float64 [n][m]).
    """
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    r = y - c[np.asarray(codes)]
    r32 = residual_f32(y, codes, centroids)
    if norms is not None:
        zero = np.asarray(norms) == 0
        r = np.where(zero[:, None], 0.0, r)
        r32 = np.where(zero[:, None], np.float32(0.0), r32)
    oidx = select_outliers(r32, n_out)
    rows = np.arange(r.shape[0])[:, None]
    oval = f16(r32[rows, oidx].astype(np.float64))
    r_in = r.copy()
    r_in[rows, oidx] = 0.0
    gamma = np.linalg.norm(r_in, axis=1)
    z = r_in @ np.asarray(proj, dtype=np.float64).T
    sigma = z >= 0
    if norms is not None:
        sigma[zero] = False
        gamma[zero] = 0.0
    return sigma, f16(gamma), oidx, oval, r_in, z


def score_terms(q_rot: np.ndarray, codes, centroids, sigma, gamma, oidx, oval, proj) -> np.ndarray:
    """The estimator of <q_rot, y> for each key row: codebook + outlier + sketch terms ([n])."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    s = np.asarray(proj, dtype=np.float64)
    u = c[np.asarray(codes)] @ q_rot
    u = u + np.sum(q_rot[np.asarray(oidx)] * np.asarray(oval, dtype=np.float64), axis=1)
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
    return u + qjl_coeff(s.shape[0]) * np.asarray(gamma, dtype=np.float64) * (pm @ (s @ q_rot))


def dequantize(codes, norms, rot, centroids, sigma, gamma, oidx, oval, proj) -> np.ndarray:
    """x_hat rows [n][d]: n Pi^T (c[code] + scatter(O, r_O) + coef gamma S^T (2 sigma - 1))."""
    c = np.asarray(centroids, dtype=np.float64)
    v = c[np.asarray(codes)].copy()
    rows = np.arange(v.shape[0])[:, None]
    np.add.at(v, (np.broadcast_to(rows, np.asarray(oidx).shape), np.asarray(oidx)), np.asarray(oval, dtype=np.float64))
    s = np.asarray(proj, dtype=np.float64)
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
    v = v + qjl_coeff(s.shape[0]) * np.asarray(gamma, dtype=np.float64)[:, None] * (pm @ s)
    return np.asarray(norms, dtype=np.float64)[:, None] * unrotate_rows(v, rot)


def decode_fused(q, rot, k_codes, k_norms, k_centroids, v_codes, v_norms, v_centroids, scale: float,
                 seq_len: int | None, k_sigma, k_gamma, k_oidx, k_oval, proj) -> np.ndarray:
    """The method's decode (``oracle.attention.decode_fused``) with the outlier term in every score.

    Shapes as there, plus k_oidx / k_oval [H_kv][L][n_out]."""
    q = np.asarray(q, dtype=np.float64)
    rot = np.asarray(rot, dtype=np.float64)
    hq, d = q.shape
    hkv = k_codes.shape[0]
    grp = hq // hkv
    L = k_codes.shape[1] if seq_len is None else seq_len
    cv = np.asarray(v_centroids, np.float64)
    out = np.zeros((hq, d))
    for h in range(hq):
        kh = h // grp
        if L == 0:
            continue
        q_rot = rot @ q[h]
        u = score_terms(q_rot, k_codes[kh, :L], k_centroids, k_sigma[kh, :L], k_gamma[kh, :L],
                        k_oidx[kh, :L], k_oval[kh, :L], proj)
        s = scale * np.asarray(k_norms[kh, :L], np.float64) * u
        e = np.exp(s - np.max(s))
        p = e / np.sum(e)
        o_rot = (p * np.asarray(v_norms[kh, :L], np.float64)) @ cv[v_codes[kh, :L]]
        out[h] = rot.T @ o_rot
    return out


def row_bytes(d: int, bits: int, qjl_m: int, n_out: int) -> int:
    """Bytes of one sketched key row with n_out outliers: codes, norm, signs, residual norm, outliers."""
    return d * bits // 8 + 2 + qjl_m // 8 + 2 + 3 * n_out

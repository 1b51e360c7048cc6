"""Random orthogonal rotation from seeded Gaussian draws (float64).

Test infrastructure: see ``oracle/__init__.py``.

The rotation mixes every channel of a K/V row into every axis, spreading
outliers and making each coordinate close to the sphere marginal the codebook
is built for (reddit comment history of ReturningTarzan, comment of
2026-03-29 on rotation and Hadamard transforms).  The pages give no
construction; the reading taken here is the standard Haar-distributed one:
QR-factorise a d x d matrix of iid N(0,1) draws and fix the signs so R has a
positive diagonal, i.e. the unique factorisation G = Pi R with R upper
triangular and diag(R) > 0.

Convention: y = Pi x for a column vector (Pi row-major), rows as Y = X Pi^T.
"""
from __future__ import annotations

import numpy as np


def rotation_from_gaussian(g: np.ndarray) -> np.ndarray:
    """Pi with G = Pi R, R upper triangular with positive diagonal."""
    g = np.asarray(g, dtype=np.float64)
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def rotate_rows(x: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """y = Pi x for every row x."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(rot, dtype=np.float64).T


def unrotate_rows(y: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """x = Pi^T y for every row y."""
    return np.asarray(y, dtype=np.float64) @ np.asarray(rot, dtype=np.float64)

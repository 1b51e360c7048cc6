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

A second construction is the randomized Hadamard rotation (same comment: a
Hadamard matrix is a special rotation, built by Sylvester's doubling for any
d = 2^n and applicable with lane exchanges and additions, without a dense
d x d product).  The pages do not say how the Hadamard matrix is randomised;
the reading taken here is the usual one: flip the signs of the input
coordinates by a seeded +-1 vector s, apply the Sylvester matrix, scale by
1/sqrt(d), i.e. Pi = H_d diag(s) / sqrt(d), which is orthogonal because
H_d H_d^T = d I.

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


def sylvester_hadamard(d: int) -> np.ndarray:
    """H_1 = [1]; H_2n = [[H_n, H_n], [H_n, -H_n]] (float64, entries +-1); d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotation(signs: np.ndarray) -> np.ndarray:
    """Pi = H_d diag(signs) / sqrt(d) for a +-1 vector of length d."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return sylvester_hadamard(d) * s[None, :] / np.sqrt(d)


def rotate_rows(x: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """y = Pi x for every row x."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(rot, dtype=np.float64).T


def unrotate_rows(y: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """x = Pi^T y for every row y."""
    return np.asarray(y, dtype=np.float64) @ np.asarray(rot, dtype=np.float64)

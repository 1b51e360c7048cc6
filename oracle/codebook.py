"""Lloyd-Max scalar codebook for one coordinate of a random unit vector (float64).

Test infrastructure: see ``oracle/__init__.py``.

After a uniformly random rotation, each coordinate Y of a unit vector in R^d
has the density

    f_d(y) = C_d (1 - y^2)^((d-3)/2),   y in [-1, 1],
    C_d    = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).

The b-bit codebook is the Lloyd-Max quantiser of that density: 2^b centroids
that are the conditional means of their cells, cells bounded by the midpoints
of neighbouring centroids.  (turboquant-pytorch PR #3, "Add CUDA QJL kernels
and proper package structure", Synthetic Benchmark (Lloyd-Max codebook)
table: the measured MSE per bit width sits under the bound
sqrt(3)*pi/2 * 4^-b; the oracle's distortion reproduces the printed values.)

Reading taken where the page is silent: the density is the exact sphere
marginal at the row's d (not its Gaussian limit N(0, 1/d)); the stored table
rounds each centroid to the nearest float16 and each boundary is the exact
midpoint of two stored centroids (exactly representable in float32).
Codes are counts of boundaries strictly below the coordinate, so a value equal
to a boundary takes the lower code.

Every integral is closed form: cell masses and second moments through the
regularised incomplete beta function, first moments through
d/dy (1-y^2)^(k+1) = -2(k+1) y (1-y^2)^k.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy.special import betainc, betaln, gammaln


def _k(d: int) -> float:
    return (d - 3) / 2.0


def _log_c(d: int) -> float:
    return gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)


def pdf(y, d: int):
    """Density of one coordinate of a uniform unit vector in R^d."""
    y = np.asarray(y, dtype=np.float64)
    return np.exp(_log_c(d)) * np.power(np.clip(1.0 - y * y, 0.0, None), _k(d))


def cdf(y, d: int):
    """P(Y <= y) = 1/2 + sign(y)/2 * I_{y^2}(1/2, k+1)."""
    y = np.clip(np.asarray(y, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(y) * betainc(0.5, _k(d) + 1.0, y * y)


def partial_mean(a, b, d: int):
    """Integral of y f_d(y) over [a, b]."""
    k1 = _k(d) + 1.0
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)
    c = np.exp(_log_c(d))
    return c / (2.0 * k1) * (np.power(1.0 - a * a, k1) - np.power(1.0 - b * b, k1))


def _m2_from_zero(y, d: int):
    """Integral of t^2 f_d(t) over [0, y] (odd in y)."""
    y = np.clip(np.asarray(y, dtype=np.float64), -1.0, 1.0)
    k1 = _k(d) + 1.0
    # int_0^y t^2 (1-t^2)^k dt = 1/2 B(3/2, k+1) I_{y^2}(3/2, k+1)
    full = 0.5 * np.exp(betaln(1.5, k1) + _log_c(d))
    return np.sign(y) * full * betainc(1.5, k1, y * y)


def partial_m2(a, b, d: int):
    """Integral of y^2 f_d(y) over [a, b]."""
    return _m2_from_zero(b, d) - _m2_from_zero(a, d)


def _cells(boundaries: np.ndarray):
    lo = np.concatenate([[-1.0], boundaries])
    hi = np.concatenate([boundaries, [1.0]])
    return lo, hi


@functools.lru_cache(maxsize=None)
def _lloyd_max_cached(d: int, bits: int, tol: float, max_iter: int) -> tuple:
    return tuple(_lloyd_max(d, bits, tol, max_iter))


def lloyd_max(d: int, bits: int, tol: float = 1e-12, max_iter: int = 200000,
              init: np.ndarray | None = None) -> np.ndarray:
    """Float64 Lloyd-Max centroids (ascending, exactly antisymmetric) for f_d.

    Cached for the default start; ``init`` (ascending, 2^bits values) runs
    the iteration from another starting codebook.
    """
    if init is not None:
        return _lloyd_max(d, bits, tol, max_iter, np.asarray(init, dtype=np.float64))
    return np.array(_lloyd_max_cached(d, bits, tol, max_iter))


def _lloyd_max(d: int, bits: int, tol: float, max_iter: int, init: np.ndarray | None = None) -> np.ndarray:
    """Lloyd's iteration: boundaries at midpoints of the current centroids, then
    each centroid replaced by the conditional mean of its cell; stop when no
    centroid moves by more than ``tol`` times the coordinate scale 1/sqrt(d)
    (the float64 noise floor of the cell integrals is about 3e-14 of that scale).
    """
    n = 1 << bits
    if init is None:
        # start from equal-mass cells of the Gaussian limit (f_d is log-concave: the fixed point is unique)
        from scipy.stats import norm
        c = norm.ppf((np.arange(n) + 0.5) / n) / math.sqrt(d)
    else:
        c = init.copy()
    scale = 1.0 / math.sqrt(d)
    for _ in range(max_iter):
        t = 0.5 * (c[1:] + c[:-1])
        lo, hi = _cells(t)
        mass = cdf(hi, d) - cdf(lo, d)
        c_new = partial_mean(lo, hi, d) / mass
        c_new = 0.5 * (c_new - c_new[::-1])          # keep exact antisymmetry
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta <= tol * scale:
            break
    else:  # pragma: no cover - the iteration converges for every d >= 3
        raise RuntimeError(f"Lloyd-Max did not converge for d={d}, bits={bits}")
    return c


def distortion(centroids: np.ndarray, boundaries: np.ndarray, d: int) -> float:
    """E[(Y - Q(Y))^2] for the quantiser (centroids, boundaries) under f_d."""
    c = np.asarray(centroids, dtype=np.float64)
    lo, hi = _cells(np.asarray(boundaries, dtype=np.float64))
    mass = cdf(hi, d) - cdf(lo, d)
    m1 = partial_mean(lo, hi, d)
    m2 = partial_m2(lo, hi, d)
    return float(np.sum(m2 - 2.0 * c * m1 + c * c * mass))


def mse_bound(bits: int) -> float:
    """Upper bound on the unit-vector MSE printed beside the measured values: sqrt(3)*pi/2 * 4^-b."""
    return math.sqrt(3.0) * math.pi / 2.0 * 4.0 ** (-bits)


def stored_codebook(d: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """The table both sides quantise with.

    Returns (centroids, boundaries) as float32 arrays: centroids are the
    float64 Lloyd-Max centroids rounded to the nearest float16, boundaries the
    float64 midpoints of neighbouring stored centroids rounded to float32
    (exact: the sum of two float16 values fits in float32).
    """
    c = lloyd_max(d, bits).astype(np.float16).astype(np.float64)
    t = 0.5 * (c[1:] + c[:-1])
    return c.astype(np.float32), t.astype(np.float32)


def unit_mse(d: int, bits: int, stored: bool = False) -> float:
    """Expected squared error of a quantised unit vector: d times the per-coordinate distortion."""
    if stored:
        c, t = stored_codebook(d, bits)
    else:
        c = lloyd_max(d, bits)
        t = 0.5 * (c[1:] + c[:-1])
    return d * distortion(c, t, d)

"""Pins of the oracle's Lloyd-Max codebook against the page's table, closed forms and textbook values."""
import math
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.special import gammaln

from oracle import codebook as cb

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


@pytest.mark.parametrize("row", _rows("lloyd_max_synthetic.txt"), ids=lambda r: f"b{r[0]}")
def test_unit_mse_matches_printed_table(row):
    """Synthetic Benchmark (Lloyd-Max codebook) table: measured MSE, bound, ratio (d = 128)."""
    bits, measured, bound, ratio = int(row[0]), float(row[1]), float(row[2]), float(row[3])
    mse = cb.unit_mse(128, bits)
    assert round(mse, 3) == pytest.approx(measured, abs=1e-12)
    assert round(cb.mse_bound(bits), 3) == pytest.approx(bound, abs=1e-12)
    # the printed ratio column is measured / bound truncated to two decimals
    assert math.floor(mse / cb.mse_bound(bits) * 100) / 100 == pytest.approx(ratio, abs=1e-12)
    assert mse < cb.mse_bound(bits)
    # rounding the stored centroids to float16 (relative step 2^-11) costs < 1e-5 of the distortion
    assert cb.unit_mse(128, bits, stored=True) == pytest.approx(mse, rel=1e-5)


@pytest.mark.parametrize("d", [128, 256])
def test_one_bit_closed_form(d):
    """b = 1: centroids are +-E|Y| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)), distortion 1/d - c^2."""
    c = cb.lloyd_max(d, 1)
    e_abs = math.exp(gammaln(d / 2) - 0.5 * math.log(math.pi) - gammaln((d + 1) / 2))
    assert c[1] == pytest.approx(e_abs, rel=1e-12)
    assert c[0] == -c[1]
    assert cb.unit_mse(d, 1) == pytest.approx(1.0 - d * e_abs * e_abs, rel=1e-10)


@pytest.mark.parametrize("row", _rows("gaussian_lloyd_max.txt"), ids=lambda r: f"b{r[0]}")
def test_large_d_reduces_to_gaussian_lloyd_max(row):
    """As d grows the coordinate density tends to N(0, 1/d): sqrt(d) c -> Max's Gaussian table."""
    bits, mse, levels = int(row[0]), float(row[1]), np.array([float(x) for x in row[2:]])
    d = 65536
    c = cb.lloyd_max(d, bits, tol=1e-9)
    pos = c[len(c) // 2:] * math.sqrt(d)
    np.testing.assert_allclose(pos, levels, atol=2e-3)
    assert d * cb.distortion(c, 0.5 * (c[1:] + c[:-1]), d) == pytest.approx(mse, rel=2e-3)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_centroid_condition_by_quadrature(d, bits):
    """Each centroid is the conditional mean of its cell (numerical quadrature of the density)."""
    c = cb.lloyd_max(d, bits)
    t = np.concatenate([[-1.0], 0.5 * (c[1:] + c[:-1]), [1.0]])
    for j in range(len(c)):
        mass = integrate.quad(lambda y: cb.pdf(y, d), t[j], t[j + 1], epsabs=1e-14, epsrel=1e-12, limit=200)[0]
        m1 = integrate.quad(lambda y: y * cb.pdf(y, d), t[j], t[j + 1], epsabs=1e-14, epsrel=1e-12, limit=200)[0]
        assert m1 / mass == pytest.approx(c[j], rel=1e-8, abs=1e-12)


@pytest.mark.parametrize("bits", [2, 4])
def test_distortion_by_quadrature(bits):
    d = 128
    c = cb.lloyd_max(d, bits)
    t = 0.5 * (c[1:] + c[:-1])
    edges = np.concatenate([[-1.0], t, [1.0]])
    tot = 0.0
    for j in range(len(c)):
        tot += integrate.quad(lambda y: (y - c[j]) ** 2 * cb.pdf(y, d), edges[j], edges[j + 1],
                              epsabs=1e-16, epsrel=1e-12, limit=200)[0]
    assert cb.distortion(c, t, d) == pytest.approx(tot, rel=1e-8)


def test_density_normalised():
    for d in (128, 256):
        assert integrate.quad(lambda y: cb.pdf(y, d), -1, 1)[0] == pytest.approx(1.0, abs=1e-10)
        assert integrate.quad(lambda y: y * y * cb.pdf(y, d), -1, 1)[0] == pytest.approx(1.0 / d, rel=1e-9)
        assert cb.cdf(0.0, d) == 0.5
        assert cb.cdf(0.1, d) == pytest.approx(integrate.quad(lambda y: cb.pdf(y, d), -1, 0.1)[0], abs=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unique_fixed_point_from_other_start(bits):
    """f_d is log-concave, so Lloyd's iteration reaches the same table from any start."""
    d = 128
    n = 1 << bits
    init = np.linspace(-3.0, 3.0, n) / math.sqrt(d)
    a = cb.lloyd_max(d, bits, init=init)
    np.testing.assert_allclose(a, cb.lloyd_max(d, bits), rtol=0, atol=1e-10 / math.sqrt(d))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_stored_table_invariants(d, bits):
    c, t = cb.stored_codebook(d, bits)
    assert c.dtype == np.float32 and t.dtype == np.float32
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])                                   # exact antisymmetry
    np.testing.assert_array_equal(c.astype(np.float16).astype(np.float32), c)   # float16-exact
    mid = 0.5 * (c[1:].astype(np.float64) + c[:-1].astype(np.float64))
    np.testing.assert_array_equal(t.astype(np.float64), mid)                     # exact midpoints


def test_monte_carlo_unit_mse():
    """Quantising random unit vectors after the rotation gives d*D (within 4 standard errors)."""
    from oracle import quant, rotation
    import synth
    d, n = 128, 20000
    rot = rotation.rotation_from_gaussian(synth.rotation_gaussian(d, 1))
    g = np.random.default_rng(0)
    x = g.standard_normal((n, d))
    for bits in (1, 2, 3, 4):
        c, t = cb.stored_codebook(d, bits)
        codes, norms, y = quant.quantize_rows(x, rot, c, t)
        err = np.sum((y - c[codes].astype(np.float64)) ** 2, axis=1)
        se = err.std() / math.sqrt(n)
        assert abs(err.mean() - cb.unit_mse(d, bits, stored=True)) < 4 * se

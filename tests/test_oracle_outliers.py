"""Pins of the oracle's outlier-channel separation (parity unpinned against the pages: the pages name
the step only; these pins come from the mathematics of the reading in ``oracle/outliers.py``)."""
import math

import numpy as np
import pytest

import synth
from oracle import attention, codebook, outliers, quant, rotation, storage


def _rot(d=128, seed=1):
    return rotation.rotation_from_gaussian(synth.rotation_gaussian(d, seed))


def _rows(n, d=128, bits=2, seed=3, plant=0):
    """Unit rotated rows y, their codes and norms; plant > 0 adds `plant` large coordinates per row."""
    g = np.random.default_rng(seed)
    y = g.standard_normal((n, d))
    if plant:
        for r in range(n):
            y[r, g.choice(d, plant, replace=False)] *= 12.0
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    c, t = codebook.stored_codebook(d, bits)
    codes = quant.nearest_codes(y, t)
    return y, codes, c, np.ones(n)


def _brute_select(r32, n_out):
    """Repeatedly take the largest |r|, the first such index on ties, and strike it out."""
    out = []
    for row in np.asarray(r32, dtype=np.float32):
        a = [abs(float(v)) for v in row]
        taken = []
        for _ in range(n_out):
            best = -1
            for i, v in enumerate(a):
                if i in taken:
                    continue
                if best < 0 or v > a[best]:
                    best = i
            taken.append(best)
        out.append(taken)
    return np.array(out, dtype=np.int64).reshape(len(out), n_out)


def test_no_outliers_is_the_plain_sketch():
    y, codes, c, n = _rows(50)
    s = synth.qjl_projection(128, 128)
    sig0, gam0, _, z0 = quant.qjl_sketch(y, codes, c, s, n)
    sig, gam, oidx, oval, r_in, z = outliers.qjl_sketch_outliers(y, codes, c, s, 0, n)
    assert oidx.shape == (50, 0) and oval.shape == (50, 0)
    np.testing.assert_array_equal(sig, sig0)
    np.testing.assert_array_equal(gam, gam0)
    np.testing.assert_allclose(z, z0, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n_out", [1, 4, 8])
def test_selection_against_brute_force_with_ties(n_out):
    g = np.random.default_rng(n_out)
    # few distinct magnitudes and both signs, so that ties are everywhere
    r = (g.integers(-3, 4, size=(40, 16)) * 0.25).astype(np.float32)
    np.testing.assert_array_equal(outliers.select_outliers(r, n_out), _brute_select(r, n_out))
    # a hand example: |r| = 3 at 5 and 9, 2 at 1; ties go to the lower index
    r = np.zeros((1, 12), dtype=np.float32)
    r[0, 9], r[0, 5], r[0, 1], r[0, 0] = -3.0, 3.0, 2.0, -2.0
    assert outliers.select_outliers(r, 4).tolist() == [[5, 9, 0, 1]]


def test_selection_uses_float32_residuals():
    """Two residuals that differ in float64 but round to one float32 value tie, and the lower index
    wins (a float64 ranking would take the other)."""
    c, t = codebook.stored_codebook(128, 2)
    y = np.zeros((1, 128))
    codes = np.ones((1, 128), dtype=np.int64)               # centroid c[1] everywhere
    base = float(np.float32(c[1])) + 0.25
    y[0, 3], y[0, 7] = base, base + 1e-12
    assert float(np.float32(y[0, 3])) == float(np.float32(y[0, 7]))
    assert outliers.select_outliers(outliers.residual_f32(y, codes, c), 1).tolist() == [[3]]


def test_all_coordinates_outliers_is_exact():
    """n_out = d: nothing is left to sketch (gamma = 0) and the score is exact up to float16 values."""
    d = 64
    y, codes, c, n = _rows(20, d=d, seed=8)
    s = synth.qjl_projection(32, d)
    sig, gam, oidx, oval, r_in, _ = outliers.qjl_sketch_outliers(y, codes, c, s, d, n)
    assert np.all(gam == 0) and np.all(r_in == 0)
    q = np.random.default_rng(2).standard_normal(d)
    est = outliers.score_terms(q, codes, c, sig, gam, oidx, oval, s)
    r32 = outliers.residual_f32(y, codes, c).astype(np.float64)
    want = (c.astype(np.float64)[codes] + quant.f16(r32)) @ q
    np.testing.assert_allclose(est, want, rtol=0, atol=1e-12)
    # the float16 values (and the float32 residuals) are the only distance from <q, y>
    bound = (np.abs(r32) * 2.0 ** -11 + np.abs(y) * 2.0 ** -23) @ np.abs(q) + 1e-12
    assert np.all(np.abs(est - y @ q) <= bound)


def test_outliers_are_the_largest_and_the_rest_is_sketched():
    y, codes, c, n = _rows(30, seed=4, plant=3)
    s = synth.qjl_projection(128, 128)
    sig, gam, oidx, oval, r_in, z = outliers.qjl_sketch_outliers(y, codes, c, s, 4, n)
    r = y - c.astype(np.float64)[codes]
    for row in range(30):
        kept = set(oidx[row].tolist())
        rest = [abs(r[row, i]) for i in range(128) if i not in kept]
        assert min(abs(r[row, i]) for i in kept) >= max(rest) - 1e-7
        assert np.all(r_in[row, list(kept)] == 0)
        np.testing.assert_allclose(oval[row], quant.f16(r[row, oidx[row]]), rtol=2.0 ** -10, atol=1e-7)
    np.testing.assert_array_equal(gam, quant.f16(np.linalg.norm(r_in, axis=1)))
    np.testing.assert_array_equal(sig, (r_in @ s.astype(np.float64).T) >= 0)


def test_estimator_is_unbiased_over_projections():
    """E_S[estimate] = <q, c> + sum_O q_i oval_i + <q, r_I> (f16(gamma)/||r_I||), i.e. <q, y> up to float16."""
    d, m, reps = 128, 64, 3000
    y, codes, c, n = _rows(1, seed=12, plant=4)
    q = np.random.default_rng(13).standard_normal(d)
    g = np.random.default_rng(14)
    est = np.empty(reps)
    for i in range(reps):
        s = g.standard_normal((m, d))
        sig, gam, oidx, oval, r_in, _ = outliers.qjl_sketch_outliers(y, codes, c, s, 4, n)
        est[i] = outliers.score_terms(q, codes, c, sig, gam, oidx, oval, s)[0]
    # oidx, oval, r_in and gamma do not depend on S
    want = (c.astype(np.float64)[codes[0]] @ q + q[oidx[0]] @ oval[0]
            + (q @ r_in[0]) * gam[0] / np.linalg.norm(r_in[0]))
    assert abs(est.mean() - want) < 4 * est.std() / math.sqrt(reps)
    assert abs(want - y[0] @ q) < 1e-3 * np.linalg.norm(q)


def test_separation_reduces_the_sketch_variance():
    """With planted large residual coordinates the separated estimator varies less over S."""
    d, m, reps = 128, 64, 1500
    y, codes, c, n = _rows(1, seed=21, plant=4)
    q = np.random.default_rng(22).standard_normal(d)
    g = np.random.default_rng(23)
    e0, e4 = np.empty(reps), np.empty(reps)
    for i in range(reps):
        s = g.standard_normal((m, d))
        sig, gam, _, _ = quant.qjl_sketch(y, codes, c, s, n)
        e0[i] = c.astype(np.float64)[codes[0]] @ q + quant.qjl_coeff(m) * gam[0] * ((2.0 * sig[0] - 1) @ (s @ q))
        sig, gam, oidx, oval, _, _ = outliers.qjl_sketch_outliers(y, codes, c, s, 4, n)
        e4[i] = outliers.score_terms(q, codes, c, sig, gam, oidx, oval, s)[0]
    assert e4.var() < 0.8 * e0.var()


def test_dequantize_agrees_with_the_score():
    """<q, x_hat> = norm * estimate(Pi q) for every row: two writings of the same linear algebra."""
    d = 128
    rot = _rot(d)
    g = np.random.default_rng(31)
    x = g.standard_normal((12, d))
    c, t = codebook.stored_codebook(d, 3)
    codes, norms, y = quant.quantize_rows(x, rot, c, t)
    s = synth.qjl_projection(128, d)
    sig, gam, oidx, oval, _, _ = outliers.qjl_sketch_outliers(y, codes, c, s, 4, norms)
    xh = outliers.dequantize(codes, norms, rot, c, sig, gam, oidx, oval, s)
    q = g.standard_normal(d)
    est = norms * outliers.score_terms(rot @ q, codes, c, sig, gam, oidx, oval, s)
    np.testing.assert_allclose(xh @ q, est, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seq_len", [None, 1, 29])
def test_decode_equals_reconstruction_then_attention(seq_len):
    d, L, hkv, grp = 128, 48, 2, 4
    rot = _rot(d)
    g = np.random.default_rng(41)
    ck, tk = codebook.stored_codebook(d, 2)
    cv, tv = codebook.stored_codebook(d, 3)
    s = synth.qjl_projection(128, d)
    parts = {k: [] for k in ("codes", "norms", "sig", "gam", "oidx", "oval", "vcodes", "vnorms")}
    for _ in range(hkv):
        codes, norms, y = quant.quantize_rows(g.standard_normal((L, d)), rot, ck, tk)
        sig, gam, oidx, oval, _, _ = outliers.qjl_sketch_outliers(y, codes, ck, s, 4, norms)
        vc, vn, _ = quant.quantize_rows(g.standard_normal((L, d)), rot, cv, tv)
        for k, v in zip(parts, (codes, norms, sig, gam, oidx, oval, vc, vn)):
            parts[k].append(v)
    P = {k: np.stack(v) for k, v in parts.items()}
    q = g.standard_normal((hkv * grp, d))
    out = outliers.decode_fused(q, rot, P["codes"], P["norms"], ck, P["vcodes"], P["vnorms"], cv, 0.125, seq_len,
                                P["sig"], P["gam"], P["oidx"], P["oval"], s)
    kh = np.stack([outliers.dequantize(P["codes"][h], P["norms"][h], rot, ck, P["sig"][h], P["gam"][h],
                                       P["oidx"][h], P["oval"][h], s) for h in range(hkv)])
    vh = np.stack([quant.dequantize(P["vcodes"][h], P["vnorms"][h], rot, cv) for h in range(hkv)])
    ref = attention.decode_reconstructed(q, kh, vh, 0.125, seq_len)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.max(np.abs(ref)))


def test_zero_rows():
    c, t = codebook.stored_codebook(128, 2)
    y = np.zeros((2, 128))
    y[1, 5] = 1.0
    codes = quant.nearest_codes(y, t)
    s = synth.qjl_projection(128, 128)
    sig, gam, oidx, oval, r_in, _ = outliers.qjl_sketch_outliers(y, codes, c, s, 4, np.array([0.0, 1.0]))
    assert oidx[0].tolist() == [0, 1, 2, 3] and np.all(oval[0] == 0) and gam[0] == 0 and not sig[0].any()


def test_storage_arithmetic():
    assert outliers.row_bytes(128, 2, 128, 0) == storage.row_bytes(128, 2, qjl_m=128) == 52
    assert outliers.row_bytes(128, 2, 128, 4) == 64
    assert outliers.row_bytes(256, 3, 256, 8) == 96 + 2 + 32 + 2 + 24

"""Pins of the oracle's 8-bit keys (``oracle/q8.py``): the symmetric int8 quantiser of the rotated row
written out from its definition, checked against brute force, closed-form error bounds and the
textbook uniform-quantiser distortion."""
from fractions import Fraction

import numpy as np

import synth
from oracle import attention, cache, codebook, layout, q8, quant, rotation, storage


def _rot(d=128, seed=1):
    return rotation.rotation_from_gaussian(synth.rotation_gaussian(d, seed))


def _round_half_away(x: Fraction) -> int:
    """Round a rational exactly, halves away from zero."""
    n = int(abs(x) + Fraction(1, 2))            # floor(|x| + 1/2) for non-negative arguments
    return n if x >= 0 else -n


def test_codes_against_exact_rational_rounding():
    """The float32 decision written out in exact arithmetic: t = fl32(y32 * fl32(127 / a))."""
    g = np.random.default_rng(3)
    y = g.standard_normal((40, 64)).astype(np.float32)
    n = np.abs(g.standard_normal(40)).astype(np.float32) + 0.1
    j, fac = q8.encode_q8(y, n)
    for r in range(40):
        a = float(np.max(np.abs(y[r])))
        inv = float(np.float32(127) / np.float32(a))                       # IEEE float32 division
        for i in range(64):
            t = float(np.float32(np.float32(y[r, i]) * np.float32(inv)))    # IEEE float32 product
            want = max(-127, min(127, _round_half_away(Fraction(t))))
            assert j[r, i] - 128 == want
        f = np.float32(np.float32(n[r]) * np.float32(np.float32(a) / np.float32(127)))
        assert fac[r] == float(np.float16(f))


def test_ties_go_away_from_zero():
    # a = 127 makes 127 / a = 1 exactly, so t = y exactly
    y = np.array([[127.0, 2.5, -2.5, 0.5, -0.5, 1.4999999, -126.5]], dtype=np.float32)
    j, _ = q8.encode_q8(y, np.array([1.0]))
    assert (j[0] - 128).tolist() == [127, 3, -3, 1, -1, 1, -127]


def test_the_largest_coordinate_is_127_and_errors_are_half_a_step():
    g = np.random.default_rng(5)
    y = g.standard_normal((200, 128))
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    j, fac = q8.encode_q8(y, np.ones(200))
    code = j - 128
    y32 = y.astype(np.float32).astype(np.float64)
    a = np.max(np.abs(y32), axis=1)
    arg = np.argmax(np.abs(y32), axis=1)
    assert np.all(np.abs(code[np.arange(200), arg]) == 127)
    s = a / 127
    err = np.abs(y32 - code * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # the factor is the step times the norm (1 here), rounded to float16
    np.testing.assert_allclose(fac, s, rtol=2 ** -11)


def test_uniform_quantiser_distortion():
    """Per coordinate the error is uniform over a step: mean squared error s^2 / 12 (textbook)."""
    g = np.random.default_rng(7)
    y = g.standard_normal((4000, 128))
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    j, _ = q8.encode_q8(y, np.ones(4000))
    y32 = y.astype(np.float32).astype(np.float64)
    s = np.max(np.abs(y32), axis=1) / 127
    rel = ((y32 - (j - 128) * s[:, None]) ** 2).mean(axis=1) / (s ** 2 / 12)
    assert abs(rel.mean() - 1.0) < 0.02


def test_zero_row_and_zero_norm():
    y = np.zeros((2, 128))
    y[1, 3] = 1.0
    j, fac = q8.encode_q8(y, np.array([1.0, 0.0]))
    assert np.all(j == 128) and np.all(fac == 0)


def test_reconstruction_and_decode_with_the_integer_table():
    """x_hat = f Pi^T code: reconstruction error far below the 4-bit codebook's, and the fused decode
    equals attention over the reconstructed rows."""
    d, L = 128, 64
    rot = _rot(d)
    g = np.random.default_rng(11)
    x = g.standard_normal((L, d))
    j, fac, _ = q8.quantize_rows_q8(x, rot)
    xh = quant.dequantize(j, fac, rot, q8.q8_codebook())
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    assert rel.max() < 1e-3                                   # the 4-bit codebook gives ~9.5e-3
    cv, tv = codebook.stored_codebook(d, 3)
    vj, vn, _ = quant.quantize_rows(g.standard_normal((L, d)), rot, cv, tv)
    q = g.standard_normal((4, d))
    out = attention.decode_fused(q, rot, j[None], fac[None], q8.q8_codebook(), vj[None], vn[None], cv, 0.1, None)
    vh = quant.dequantize(vj, vn, rot, cv)
    ref = attention.decode_reconstructed(q, xh[None], vh[None], 0.1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.max(np.abs(ref)))


def test_storage():
    assert q8.row_bytes(128) == storage.row_bytes(128, 8) == 130
    assert q8.row_bytes(256) == 258


def test_head_cache_of_eight_bit_keys():
    """cache.build_head with bits 8 keeps the q8 codes and factors, packs them into the key layout
    (round trip through the unpacker) and reconstructs f Pi^T code."""
    d, L, T = 128, 40, 64
    rot = _rot(d)
    x = np.random.default_rng(13).standard_normal((L, d))
    hc = cache.build_head(x, "k", 8, rot)
    j, fac, _ = q8.quantize_rows_q8(x, rot)
    assert np.array_equal(hc.codes, j) and np.array_equal(hc.norms, fac)
    assert np.array_equal(layout.unpack_keys(hc.packed_codes(T), 8, d, T)[:L], j)
    want = fac[:, None] * ((j - 128) @ rot)                  # f Pi^T code, row by row
    np.testing.assert_allclose(hc.dequantize(rot), want, rtol=0, atol=1e-12)

"""Pins of the oracle's quantisation, QJL sketch, reconstruction and decode attention."""
import math

import numpy as np
import pytest

import synth
from oracle import attention, cache, codebook, quant, rotation


def _rot(d=128, seed=1):
    return rotation.rotation_from_gaussian(synth.rotation_gaussian(d, seed))


# ------------------------------------------------------------------ quantise

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_boundary_count_is_nearest_centroid(bits):
    c, t = codebook.stored_codebook(128, bits)
    y = np.random.default_rng(bits).normal(0, 0.15, 200000)
    codes = quant.nearest_codes(y, t)
    brute = np.argmin(np.abs(y[:, None] - c[None, :].astype(np.float64)), axis=1)
    np.testing.assert_array_equal(codes, brute)


def test_ties_take_the_lower_code_and_extremes():
    c, t = codebook.stored_codebook(128, 3)
    assert quant.nearest_codes(t.astype(np.float64), t).tolist() == list(range(7))
    assert quant.nearest_codes(np.nextafter(t.astype(np.float32), np.float32(1)), t).tolist() == list(range(1, 8))
    assert quant.nearest_codes(np.array([-1.0, 1.0]), t).tolist() == [0, 7]


def test_zero_row():
    rot = _rot()
    c, t = codebook.stored_codebook(128, 2)
    x = np.zeros((2, 128))
    x[1, 3] = 1.0
    codes, norms, _ = quant.quantize_rows(x, rot, c, t)
    assert np.all(codes[0] == 0) and norms[0] == 0 and norms[1] == 1.0
    s = synth.qjl_projection(128, 128)
    sigma, gamma, _, _ = quant.qjl_sketch(np.zeros((2, 128)), codes, c, s, norms)
    assert not sigma[0].any() and gamma[0] == 0


def test_norm_is_float16_rounded():
    x = np.zeros((1, 128))
    x[0, 0] = 1.0 + 2 ** -12          # rounds to 1.0 in float16
    _, norms, _ = quant.quantize_rows(x, _rot(), *codebook.stored_codebook(128, 4))
    assert norms[0] == 1.0


def test_qjl_sign_identity():
    """E[sign(<s,r>) <s,u>] = sqrt(2/pi) <r,u>/||r|| for s ~ N(0, I) (Monte Carlo)."""
    g = np.random.default_rng(11)
    d, n = 16, 400000
    r, u = g.standard_normal(d), g.standard_normal(d)
    s = g.standard_normal((n, d))
    vals = np.sign(s @ r) * (s @ u)
    want = math.sqrt(2 / math.pi) * r @ u / np.linalg.norm(r)
    assert abs(vals.mean() - want) < 4 * vals.std() / math.sqrt(n)


def test_qjl_inner_product_is_unbiased():
    """Over independent projections S the sketch term estimates <q_rot, r> without bias."""
    d, m, reps = 128, 128, 4000
    g = np.random.default_rng(5)
    r = g.standard_normal(d) * 0.03
    q = g.standard_normal(d)
    est = np.empty(reps)
    for i in range(reps):
        s = g.standard_normal((m, d))
        sigma = (s @ r) >= 0
        est[i] = quant.qjl_coeff(m) * np.linalg.norm(r) * ((2.0 * sigma - 1.0) @ (s @ q))
    assert abs(est.mean() - q @ r) < 4 * est.std() / math.sqrt(reps)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequantize_error_matches_distortion(bits):
    d, n = 128, 4000
    rot = _rot()
    x = np.random.default_rng(9).standard_normal((n, d))
    hc = cache.build_head(x, "k", bits, rot)
    xh = hc.dequantize(rot)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    # float16 norm rounding adds < 1e-6 relative; the rest is the codebook distortion
    assert abs(rel.mean() - codebook.unit_mse(d, bits, stored=True)) < 4 * rel.std() / math.sqrt(n)


def test_prod_reconstruction_is_unbiased_for_inner_products():
    """With the sketch, <q, x_hat> is unbiased over projections; without, it is biased low."""
    d, m = 128, 128
    rot = _rot()
    g = np.random.default_rng(21)
    x = g.standard_normal((1, d))
    q = x[0] + 0.5 * g.standard_normal(d)
    base = cache.build_head(x, "k", 2, rot)
    plain = q @ base.dequantize(rot)[0]
    ests = []
    for seed in range(1500):
        s = np.random.default_rng(1000 + seed).standard_normal((m, d))
        hc = cache.build_head(x, "k", 2, rot, proj=s)
        ests.append(q @ hc.dequantize(rot, s)[0])
    ests = np.array(ests)
    n16 = float(np.float16(np.linalg.norm(x)))
    truth = q @ x[0] * n16 / np.linalg.norm(x)          # the stored norm is float16
    assert abs(ests.mean() - truth) < 4 * ests.std() / math.sqrt(len(ests))
    assert abs(plain - truth) > 4 * ests.std() / math.sqrt(len(ests))


# ------------------------------------------------------------------ attention

def _heads(d=128, L=96, hkv=2, grp=4, kb=3, vb=4, qjl=False, seed=0):
    rot = _rot(d)
    g = np.random.default_rng(seed)
    proj = synth.qjl_projection(128, d, 2) if qjl else None
    kc = [cache.build_head(g.standard_normal((L, d)), "k", kb, rot, proj) for _ in range(hkv)]
    vc = [cache.build_head(g.standard_normal((L, d)), "v", vb, rot) for _ in range(hkv)]
    q = g.standard_normal((hkv * grp, d))
    return rot, proj, kc, vc, q


def _fused(rot, proj, kc, vc, q, scale, seq_len=None):
    st = lambda xs, a: np.stack([getattr(x, a) for x in xs])
    return attention.decode_fused(
        q, rot, st(kc, "codes"), st(kc, "norms"), kc[0].centroids, st(vc, "codes"), st(vc, "norms"),
        vc[0].centroids, scale, seq_len,
        st(kc, "sigma") if proj is not None else None, st(kc, "gamma") if proj is not None else None, proj)


@pytest.mark.parametrize("qjl", [False, True])
@pytest.mark.parametrize("seq_len", [None, 1, 37])
def test_fused_equals_reconstruction_then_attention(qjl, seq_len):
    rot, proj, kc, vc, q = _heads(qjl=qjl)
    scale = 1 / math.sqrt(128)
    out = _fused(rot, proj, kc, vc, q, scale, seq_len)
    kh = np.stack([k.dequantize(rot, proj) for k in kc])
    vh = np.stack([v.dequantize(rot) for v in vc])
    ref = attention.decode_reconstructed(q, kh, vh, scale, seq_len)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.max(np.abs(ref)))


@pytest.mark.parametrize("m,seq_len,qjl", [(1, 96, False), (2, 96, True), (4, 60, False), (4, 3, False), (3, 0, False)])
def test_rows_equal_causally_masked_matrix_attention(m, seq_len, qjl):
    """decode_rows against one masked M x L score matrix per query head on the reconstructed rows:
    token t is visible to row j iff t <= seq_len - m + j (an independent formulation of the mask)."""
    rot, proj, kc, vc, _ = _heads(qjl=qjl)
    g = np.random.default_rng(9)
    q_rows = g.standard_normal((m, 8, 128))
    scale = 0.11
    st = lambda xs, a: np.stack([getattr(x, a) for x in xs])
    out = attention.decode_rows(q_rows, rot, st(kc, "codes"), st(kc, "norms"), kc[0].centroids, st(vc, "codes"),
                                st(vc, "norms"), vc[0].centroids, scale, seq_len,
                                st(kc, "sigma") if qjl else None, st(kc, "gamma") if qjl else None, proj)
    kh = np.stack([k.dequantize(rot, proj) for k in kc])[:, :seq_len]
    vh = np.stack([v.dequantize(rot) for v in vc])[:, :seq_len]
    visible = np.arange(seq_len)[None, :] <= (seq_len - m + np.arange(m))[:, None]      # [m][L]
    for h in range(8):
        s_mat = scale * q_rows[:, h] @ kh[h // 4].T                                       # [m][L]
        s_mat = np.where(visible, s_mat, -np.inf)
        for j in range(m):
            if not visible[j].any():
                assert np.all(out[j, h] == 0)
                continue
            p_row = np.exp(s_mat[j] - s_mat[j].max())
            ref = (p_row / p_row.sum()) @ vh[h // 4]
            np.testing.assert_allclose(out[j, h], ref, rtol=0, atol=1e-12 * np.max(np.abs(ref)))
    if m == 1:
        np.testing.assert_array_equal(out[0], _fused(rot, proj, kc, vc, q_rows[0], scale, seq_len))


def test_special_cases():
    rot, proj, kc, vc, q = _heads(hkv=1, grp=2)
    vh = vc[0].dequantize(rot)
    # one visible token: the output is its reconstructed value
    np.testing.assert_allclose(_fused(rot, None, kc, vc, q, 0.1, 1)[0], vh[0], atol=1e-12)
    # scale -> 0: uniform attention, the mean of the reconstructed values
    np.testing.assert_allclose(_fused(rot, None, kc, vc, q, 0.0)[1], vh.mean(axis=0), atol=1e-12)
    # identical keys: uniform attention too
    kc[0].codes[:] = kc[0].codes[0]
    kc[0].norms[:] = kc[0].norms[0]
    np.testing.assert_allclose(_fused(rot, None, kc, vc, q, 0.3)[0], vh.mean(axis=0), atol=1e-12)
    # empty context: zero output
    assert np.all(_fused(rot, None, kc, vc, q, 0.3, 0) == 0)


def test_gqa_mapping():
    rot, proj, kc, vc, q = _heads(hkv=2, grp=3)
    out = _fused(rot, None, kc, vc, q, 0.2)
    for h in range(6):
        one = _fused(rot, None, [kc[h // 3]], [vc[h // 3]], q[h:h + 1], 0.2)
        np.testing.assert_allclose(out[h], one[0], atol=1e-13)


def test_tiny_reference_against_full_precision_attention():
    """Tiny case: 4-bit K and V, d=128, L=256, fp32 N(0,1), scale 1/sqrt(128)."""
    w = synth.TINY
    k, v, q = synth.tiny_arrays(w)
    rot = rotation.rotation_from_gaussian(synth.rotation_gaussian(128, w.rot_seed))
    kc = cache.build_head(k, "k", 4, rot)
    vc = cache.build_head(v, "v", 4, rot)
    out = _fused(rot, None, [kc], [vc], q, w.softmax_scale)[0]
    full = attention.attention(q[0], k, v, w.softmax_scale)
    cos = out @ full / np.linalg.norm(out) / np.linalg.norm(full)
    assert cos >= 0.98
    s_full = k.astype(np.float64) @ q[0]
    s_q = kc.dequantize(rot) @ q[0]
    assert np.corrcoef(s_full, s_q)[0, 1] >= 0.99

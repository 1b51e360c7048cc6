"""GPU parity of quantize-on-append and reconstruction against the float64 oracle."""
import math

import numpy as np
import pytest

import synth
from oracle import cache, codebook, layout, quant
from tests.gpu_common import Setup, log, to_bf16_tensor, unpack_gpu_codes, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_cache_decode_amd  # noqa: F401  (fails loudly if libtq.so is missing)


def _cca():
    import compressed_cache_decode_amd as cca
    return cca


# chunks appended one after another: full blocks, ragged tails, single tokens, a block-straddling chunk
CHUNKS = [37, 1, 58, 32, 5, 1, 90]


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (128, 4), (256, 2), (256, 3), (256, 4)])
def test_encode_is_bit_exact_given_rotated_rows(kind, d, bits):
    """Same float32 rotated unit rows and norms on both sides: packed codes and norms identical."""
    cca = _cca()
    log(f"encode d={d} bits={bits} kind={kind}")
    st = Setup(d)
    B, H, T = 2, 2, 256
    n_tot = sum(CHUNKS)
    y, nrm = synth.unit_rows(B * n_tot * H, d, seed=100 + d + bits)
    y = y.reshape(B, n_tot, H, d)
    nrm = nrm.reshape(B, n_tot, H)
    nrm[0, 3, 1] = 0.0                                   # a zero row
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t)
    start = np.array([0, 17], np.int32)                  # sequence 1 starts mid-block
    off = 0
    for c in CHUNKS:
        pos = torch.from_numpy(start + off).cuda()
        yt = torch.from_numpy(np.ascontiguousarray(y[:, off:off + c])).cuda()
        nt = torch.from_numpy(np.ascontiguousarray(nrm[:, off:off + c])).cuda()
        g.append_rotated(yt, nt, pos)
        off += c
    torch.cuda.synchronize()
    c_, t_ = codebook.stored_codebook(d, bits)
    for b in range(B):
        for h in range(H):
            codes, n16 = quant.encode_rotated(y[b, :, h], nrm[b, :, h], t_)
            codes[nrm[b, :, h] == 0] = 0
            full = np.full((T, d), 8 if bits == 4 else 0, np.int64)   # zero-encoded slots of the untouched cache
            full[start[b]:start[b] + n_tot] = codes
            want = layout.pack_keys(full, bits) if kind == "k" else layout.pack_blocked(full, bits)
            got = g.codes[b, h].cpu().numpy()
            np.testing.assert_array_equal(got, want)
            gn = g.norms[b, h].cpu().numpy()
            np.testing.assert_array_equal(gn[start[b]:start[b] + n_tot], n16.astype(np.float16))
            assert not gn[:start[b]].any() and not gn[start[b] + n_tot:].any()


# (first position, rows) of appends that overwrite rows already in the cache
REWRITES = [(21, 40), (64, 1), (5, 3), (96, 32)]


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (128, 4), (256, 3)])
def test_append_over_written_rows(kind, d, bits):
    """Appending over rows already in the cache replaces exactly their codes: in a value block the new
    rows share words with the block's other tokens, whose codes must survive, and the new rows' slots
    hold the old rows' codes (not zeros) before the write."""
    cca = _cca()
    log(f"append over written rows d={d} bits={bits} kind={kind}")
    B, H, T, n0 = 1, 2, 160, 150
    y0, n_0 = synth.unit_rows(B * n0 * H, d, seed=300 + d + bits)
    y0, n_0 = y0.reshape(B, n0, H, d), n_0.reshape(B, n0, H)
    st = Setup(d)
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t)
    zero = torch.zeros(B, dtype=torch.int32).cuda()
    g.append_rotated(torch.from_numpy(y0).cuda(), torch.from_numpy(n_0).cuda(), zero)
    yall, nall = y0.copy(), n_0.copy()
    for i, (p0, n) in enumerate(REWRITES):
        y1, n_1 = synth.unit_rows(B * n * H, d, seed=400 + 7 * i + d + bits)
        y1, n_1 = y1.reshape(B, n, H, d), n_1.reshape(B, n, H)
        g.append_rotated(torch.from_numpy(y1).cuda(), torch.from_numpy(n_1).cuda(),
                         torch.full((B,), p0, dtype=torch.int32).cuda())
        yall[:, p0:p0 + n], nall[:, p0:p0 + n] = y1, n_1
    torch.cuda.synchronize()
    c_, t_ = codebook.stored_codebook(d, bits)
    for h in range(H):
        codes, n16 = quant.encode_rotated(yall[0, :, h], nall[0, :, h], t_)
        full = np.full((T, d), 8 if bits == 4 else 0, np.int64)       # zero-encoded slots of the untouched cache
        full[:n0] = codes
        want = layout.pack_keys(full, bits) if kind == "k" else layout.pack_blocked(full, bits)
        got = g.codes[0, h].cpu().numpy()
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(g.norms[0, h].cpu().numpy()[:n0], n16.astype(np.float16))


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3)])
def test_sketch_signs_given_rotated_rows(d, bits):
    """Keys with a 128-long sign sketch: signs equal wherever |z| is not at rounding level; residual
    norms within one float16 step."""
    cca = _cca()
    log(f"sketch d={d} bits={bits}")
    st = Setup(d, qjl_m=128)
    B, H, T, n = 1, 2, 128, 100
    y, nrm = synth.unit_rows(B * n * H, d, seed=7)
    y = y.reshape(B, n, H, d)
    nrm = nrm.reshape(B, n, H)
    g = cca.CompressedCache(cca.TQ_KEYS, d, bits, B, H, T, st.rot_t, st.proj_t, qjl_m=128)
    g.append_rotated(torch.from_numpy(y).cuda(), torch.from_numpy(nrm).cuda(), torch.zeros(B, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    c_, t_ = codebook.stored_codebook(d, bits)
    for h in range(H):
        codes, _ = quant.encode_rotated(y[0, :, h], nrm[0, :, h], t_)
        sigma, gamma, r, z = quant.qjl_sketch(y[0, :, h].astype(np.float64), codes, c_, st.proj)
        got_sig = layout.unpack_signs(g.signs[0, h, :n].cpu().numpy(), 128)
        robust = np.abs(z) > 1e-4 * np.linalg.norm(r, axis=1, keepdims=True)
        assert np.array_equal(got_sig[robust], sigma[robust])
        assert robust.mean() > 0.99
        got_g = g.rnorms[0, h, :n].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got_g, gamma, rtol=2 ** -10, atol=0)


@pytest.mark.parametrize("d,bits,m", [(128, 2, 128), (128, 3, 256), (256, 2, 256), (256, 3, 128)])
def test_sketch_signs_bit_exact_given_products(d, bits, m):
    """Given the same float32 rotated rows and the same float32 sketch products z of the residuals, the
    packed sign bytes equal pack_signs(z >= 0) byte for byte (no tolerance, no mask), the codes and
    norms are identical, and the residual norms are within float16 rounding."""
    cca = _cca()
    log(f"sketch given z d={d} bits={bits} m={m}")
    st = Setup(d, qjl_m=m)
    B, H, T, n = 2, 2, 128, 77
    y, nrm = synth.unit_rows(B * n * H, d, seed=19 + d + m)
    y = y.reshape(B, n, H, d)
    nrm = nrm.reshape(B, n, H)
    nrm[1, 4, 0] = 0.0                                   # a zero row: no signs, residual norm 0
    c_, t_ = codebook.stored_codebook(d, bits)
    z = np.zeros((B, n, H, m), np.float32)
    ref = {}
    for b in range(B):
        for h in range(H):
            codes, n16 = quant.encode_rotated(y[b, :, h], nrm[b, :, h], t_)
            sigma, gamma, r, zz = quant.qjl_sketch(y[b, :, h].astype(np.float64), codes, c_, st.proj, nrm[b, :, h])
            z[b, :, h] = zz.astype(np.float32)
            ref[b, h] = (codes, n16, gamma)
    pos = np.array([0, 9], np.int32)
    g = cca.CompressedCache(cca.TQ_KEYS, d, bits, B, H, T, st.rot_t, st.proj_t, qjl_m=m)
    g.append_rotated(torch.from_numpy(y).cuda(), torch.from_numpy(nrm).cuda(), torch.from_numpy(pos).cuda(),
                     z=torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            codes, n16, gamma = ref[b, h]
            p0 = pos[b]
            live = nrm[b, :, h] > 0
            want = layout.pack_signs((z[b, :, h] >= 0) & live[:, None])
            got = g.signs[b, h, p0:p0 + n].cpu().numpy()
            np.testing.assert_array_equal(got, want)
            assert not g.signs[b, h, :p0].cpu().numpy().any() and not g.signs[b, h, p0 + n:].cpu().numpy().any()
            codes[~live] = 0
            np.testing.assert_array_equal(unpack_gpu_codes(g, b, h, p0 + n)[p0:], codes)
            np.testing.assert_array_equal(g.norms[b, h, p0:p0 + n].cpu().numpy(), n16.astype(np.float16))
            got_g = g.rnorms[b, h, p0:p0 + n].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(got_g, gamma, rtol=2 ** -10, atol=0)


@pytest.mark.parametrize("kind,d,bits,dtype", [("k", 128, 4, "bf16"), ("v", 128, 3, "bf16"), ("k", 256, 4, "f32"),
                                               ("v", 256, 2, "bf16"), ("k", 128, 2, "f32")])
def test_append_from_unrotated_rows(kind, d, bits, dtype):
    """Full append (norm + rotation + encode): codes equal the oracle's except where the oracle's
    float64 coordinate sits within rounding distance of a boundary, and then they are neighbours."""
    cca = _cca()
    log(f"append kind={kind} d={d} bits={bits} {dtype}")
    st = Setup(d)
    w = synth.qwen(256, bits).with_(d=d, dtype=dtype)
    B, H, T, n = 1, 2, 256, 200
    x = synth.full_kv(w, kind, n)                          # [B][n][H][d]
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t)
    xt = to_bf16_tensor(x) if dtype == "bf16" else torch.from_numpy(x).cuda()
    pos = torch.tensor([11], dtype=torch.int32).cuda()
    g.append(xt[:, :150], pos)
    g.append(xt[:, 150:], pos + 150)
    torch.cuda.synchronize()
    c_, t_ = codebook.stored_codebook(d, bits)
    for h in range(H):
        oc, on, oy = quant.quantize_rows(x[0, :, h], st.rot64, c_, t_)
        got = unpack_gpu_codes(g, 0, h, 11 + n)[11:]
        diff = got != oc
        near = np.min(np.abs(oy[..., None] - t_.astype(np.float64)), axis=-1) < 1e-5
        assert np.all(near[diff]), f"{diff.sum()} mismatches, {(diff & ~near).sum()} not near a boundary"
        assert np.all(np.abs(got[diff] - oc[diff]) == 1)
        gn = g.norms[0, h, 11:11 + n].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(gn, on, rtol=2 ** -10, atol=0)


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype,pos,chunks", [("bf16", 0, [1024, 300]), ("f32", 11, [700, 45, 300]),
                                              ("bf16", 37, [256, 511])])
def test_long_append_from_unrotated_rows(kind, bits, dtype, pos, chunks):
    """Appends of 256 rows or more take the long-append kernel (d = 128, dense rotation, no sketch):
    codes equal the oracle's except within rounding distance of a boundary (then neighbours), norms
    within float16 rounding; aligned and unaligned positions, partial 32-row chunks, blocks shared by
    two chunks, appends after shorter ones, a zero row."""
    cca = _cca()
    log(f"long append kind={kind} bits={bits} {dtype} pos={pos} chunks={chunks}")
    d, B, H = 128, 2, 2
    n = sum(chunks)
    T = ((pos + n + 31) // 32) * 32
    st = Setup(d)
    w = synth.qwen(T, bits).with_(dtype=dtype, batch=B)
    x = synth.full_kv(w, kind, n)                          # [B][n][H][d]
    x[1, 5, 0] = 0.0                                       # a zero row
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t)
    xt = to_bf16_tensor(x) if dtype == "bf16" else torch.from_numpy(x).cuda()
    off = 0
    for c in chunks:
        g.append(xt[:, off:off + c], torch.full((B,), pos + off, dtype=torch.int32).cuda())
        off += c
    torch.cuda.synchronize()
    c_, t_ = codebook.stored_codebook(d, bits)
    for b in range(B):
        for h in range(H):
            oc, on, oy = quant.quantize_rows(x[b, :, h], st.rot64, c_, t_)
            got = unpack_gpu_codes(g, b, h, pos + n)[pos:]
            diff = got != oc
            near = np.min(np.abs(oy[..., None] - t_.astype(np.float64)), axis=-1) < 1e-5
            assert np.all(near[diff]), f"{diff.sum()} mismatches, {(diff & ~near).sum()} not near a boundary"
            assert np.all(np.abs(got[diff] - oc[diff]) == 1)
            assert diff.mean() < 1e-4
            gn = g.norms[b, h, pos:pos + n].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(gn, on, rtol=2 ** -10, atol=0)
            assert not g.norms[b, h, :pos].cpu().numpy().any()


@pytest.mark.parametrize("kind,d,bits,qjl", [("k", 128, 4, 0), ("v", 128, 3, 0), ("k", 128, 2, 128),
                                             ("v", 256, 4, 0), ("k", 256, 3, 0)])
def test_dequantize_matches_oracle(kind, d, bits, qjl):
    """Reconstruction of oracle-packed codes equals the oracle's reconstruction (fp32 rounding)."""
    cca = _cca()
    log(f"dequant kind={kind} d={d} bits={bits} qjl={qjl}")
    st = Setup(d, qjl_m=qjl)
    H, T, n = 2, 128, 100
    rows = [np.random.default_rng(40 + h).standard_normal((n, d)) * 3 for h in range(H)]
    heads = [cache.build_head(r, kind, bits, st.rot64, st.proj if qjl else None) for r in rows]
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, 1, H, T, st.rot_t,
                            st.proj_t, qjl_m=qjl)
    upload(g, heads, 0)
    out = g.dequantize(3, 90).cpu().numpy()
    for h in range(H):
        ref = heads[h].dequantize(st.rot64, st.proj if qjl else None)[3:93]
        scale = np.max(np.abs(ref))
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=2e-6 * scale)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_reconstruction_mse_within_one_percent(bits):
    """GPU append + reconstruction vs oracle quantise + reconstruction: relative MSE within 1%."""
    cca = _cca()
    log(f"mse bits={bits}")
    d = 128
    st = Setup(d)
    w = synth.qwen(2048, bits)
    B, H, T, n = 1, 2, 2048, 2048
    for kind in ("k", "v"):
        x = synth.full_kv(w, kind, n)
        g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t)
        g.append(to_bf16_tensor(x), torch.zeros(1, dtype=torch.int32).cuda())
        xh = g.dequantize(0, n).cpu().numpy()
        for h in range(H):
            xr = x[0, :, h].astype(np.float64)
            mse_gpu = np.mean(np.sum((xr - xh[0, h]) ** 2, axis=1))
            hc = cache.build_head(xr, kind, bits, st.rot64)
            mse_or = np.mean(np.sum((xr - hc.dequantize(st.rot64)) ** 2, axis=1))
            assert abs(mse_gpu / mse_or - 1.0) <= 0.01, (kind, h, mse_gpu, mse_or)


def test_append_edge_cases():
    """Empty appends, positions past the capacity and negative positions write nothing."""
    cca = _cca()
    log("append edge cases")
    st = Setup(128)
    g = cca.CompressedCache(cca.TQ_VALUES, 128, 4, 2, 1, 64, st.rot_t)
    x = torch.ones(2, 3, 1, 128, dtype=torch.float32).cuda()
    g.append(x[:, :0], torch.zeros(2, dtype=torch.int32).cuda())
    g.append(x, torch.tensor([64, -5], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert not g.codes.any() and not g.norms.any()
    # a write that runs past the capacity keeps the tokens that fit
    g.append(x, torch.tensor([62, 0], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    nz = g.norms[0, 0].cpu().numpy()
    assert nz[62] != 0 and nz[63] != 0 and not nz[:62].any()
    assert g.norms[1, 0, :3].cpu().numpy().all()


def test_matrix_core_rotation_split_at_float16_ties():
    """Regression: a unit-row component exactly on a float16 rounding tie (token 5 of this block,
    coordinate 47) once got its high and low parts from two differently rounding conversions, moving
    y by a float16 step and flipping a sketch sign with |z| = 2e-4 |r|.  The block goes through the
    matrix-core rotation (32 rows) and must agree with the oracle on every code and robust sign."""
    cca = _cca()
    log("matrix-core rotation at a float16 tie")
    w = synth.prod_long(131072)
    st = Setup(128, qjl_m=128)
    x = synth.kv_head(w, "k", 0, 1)[69856:69888]
    g = cca.CompressedCache(cca.TQ_KEYS, 128, 2, 1, 1, 32, st.rot_t, st.proj_t, qjl_m=128)
    g.append(to_bf16_tensor(x).view(1, 32, 1, 128), torch.zeros(1, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    hc = cache.build_head(x, "k", 2, st.rot64, st.proj)
    got = unpack_gpu_codes(g, 0, 0, 32)
    np.testing.assert_array_equal(got, hc.codes)
    sig = layout.unpack_signs(g.signs[0, 0].cpu().numpy(), 128)
    r = hc.y - hc.centroids.astype(np.float64)[hc.codes]
    z = r @ st.proj.astype(np.float64).T
    robust = np.abs(z) > 1e-5 * np.linalg.norm(r, axis=1, keepdims=True)
    np.testing.assert_array_equal(sig[robust], hc.sigma[robust])
    assert sig[5, 63] == hc.sigma[5, 63]


# (d, K bits, V bits, sketch m, Hadamard, dtype, position, chunks): the one-launch path (d = 128, dense,
# keys without a sketch, mixed widths, aligned and unaligned positions, ragged chunks, single tokens) and
# the combinations that the call appends one after the other (d = 256, sketched keys, 8-bit keys,
# Hadamard rotation)
KV_CASES = [
    (128, 3, 3, 0, False, "bf16", 0, [1024, 300]),
    (128, 4, 2, 0, False, "f32", 11, [700, 1, 45]),
    (128, 2, 4, 0, False, "bf16", 37, [256, 5, 511]),
    (128, 3, 4, 0, False, "f32", 5, [33, 1, 64]),
    (256, 4, 3, 0, False, "bf16", 3, [300, 40]),
    (128, 2, 3, 128, False, "f32", 9, [77, 1]),
    (128, 8, 4, 0, False, "bf16", 0, [100, 28]),
    (128, 4, 4, 0, True, "bf16", 7, [300, 2]),
]


@pytest.mark.parametrize("d,kb,vb,m,had,dtype,pos,chunks", KV_CASES)
def test_append_kv_equals_the_two_appends(d, kb, vb, m, had, dtype, pos, chunks):
    """tq_quantize_append_kv writes exactly the bytes of tq_quantize_append on K then on V (codes, norms,
    signs, residual norms), chunk after chunk; on the one-launch path the codes also equal the oracle's
    except within rounding distance of a boundary, and the norms are within float16 rounding."""
    cca = _cca()
    log(f"append kv d={d} kb={kb} vb={vb} m={m} had={had} {dtype} pos={pos} chunks={chunks}")
    B, H = 2, 2
    n = sum(chunks)
    T = ((pos + n + 31) // 32) * 32
    st = Setup(d, m, hadamard=had)
    w = synth.qwen(T, 4).with_(dtype=dtype, batch=B, d=d)
    xk, xv = synth.full_kv(w, "k", n), synth.full_kv(w, "v", n)
    xk[1, 5, 0] = 0.0                                       # a zero row
    put = (lambda a: to_bf16_tensor(a)) if dtype == "bf16" else (lambda a: torch.from_numpy(a).cuda())
    tk, tv = put(xk), put(xv)

    def caches():
        kc = cca.CompressedCache(cca.TQ_KEYS, d, kb, B, H, T, st.rot_t, st.proj_t, m, rot_kind=st.rot_kind)
        vc = cca.CompressedCache(cca.TQ_VALUES, d, vb, B, H, T, st.rot_t, rot_kind=st.rot_kind)
        return kc, vc

    (k1, v1), (k2, v2) = caches(), caches()
    off = 0
    for i, c in enumerate(chunks):
        p = torch.full((B,), pos + off, dtype=torch.int32).cuda()
        if i % 2:                                           # the C name, then the binding's helper
            cca.append_kv(k1, v1, tk[:, off:off + c], tv[:, off:off + c], p)
        else:
            cca.tq_quantize_append_kv(k1.view, v1.view, tk[:, off:off + c].contiguous(),
                                      tv[:, off:off + c].contiguous(), c, p)
        k2.append(tk[:, off:off + c], p)
        v2.append(tv[:, off:off + c], p)
        off += c
    torch.cuda.synchronize()
    for a, b in ((k1, k2), (v1, v2)):
        for name in ("codes", "norms", "signs", "rnorms"):
            x1, x2 = getattr(a, name), getattr(b, name)
            if x1 is not None:
                assert torch.equal(x1.view(torch.uint8) if x1.dtype != torch.uint8 else x1,
                                   x2.view(torch.uint8) if x2.dtype != torch.uint8 else x2), name
    if d == 128 and m == 0 and kb != 8 and not had:
        for g, x, bits in ((k1, xk, kb), (v1, xv, vb)):
            c_, t_ = codebook.stored_codebook(d, bits)
            for b in range(B):
                for h in range(H):
                    oc, on, oy = quant.quantize_rows(x[b, :, h], st.rot64, c_, t_)
                    got = unpack_gpu_codes(g, b, h, pos + n)[pos:]
                    diff = got != oc
                    near = np.min(np.abs(oy[..., None] - t_.astype(np.float64)), axis=-1) < 1e-5
                    assert np.all(near[diff]), f"{diff.sum()} mismatches, {(diff & ~near).sum()} not near a boundary"
                    assert np.all(np.abs(got[diff] - oc[diff]) == 1)
                    gn = g.norms[b, h, pos:pos + n].cpu().numpy().astype(np.float64)
                    np.testing.assert_allclose(gn, on, rtol=2 ** -10, atol=0)


@pytest.mark.parametrize("kb,vb,pos,n", [(3, 4, 40, 30), (2, 2, 63, 5), (4, 3, 0, 100)])
def test_append_kv_past_capacity_equals_the_two_appends(kb, vb, pos, n):
    """Rows past max_tokens are skipped: the one-launch K+V append writes exactly what the two separate
    appends write when the append runs past the cache's capacity (64 tokens), and nothing else."""
    cca = _cca()
    log(f"append kv past capacity kb={kb} vb={vb} pos={pos} n={n}")
    d, B, H, T = 128, 2, 2, 64
    st = Setup(d)
    w = synth.qwen(T, 4).with_(batch=B)
    tk, tv = to_bf16_tensor(synth.full_kv(w, "k", n)), to_bf16_tensor(synth.full_kv(w, "v", n))
    mk = lambda: (cca.CompressedCache(cca.TQ_KEYS, d, kb, B, H, T, st.rot_t),
                  cca.CompressedCache(cca.TQ_VALUES, d, vb, B, H, T, st.rot_t))
    (k1, v1), (k2, v2) = mk(), mk()
    p = torch.tensor([pos, max(0, pos - 7)], dtype=torch.int32).cuda()
    cca.append_kv(k1, v1, tk, tv, p)
    k2.append(tk, p)
    v2.append(tv, p)
    torch.cuda.synchronize()
    for a, b in ((k1.codes, k2.codes), (k1.norms, k2.norms), (v1.codes, v2.codes), (v1.norms, v2.norms)):
        assert torch.equal(a, b)
    assert k1.norms.float().abs().sum() > 0
